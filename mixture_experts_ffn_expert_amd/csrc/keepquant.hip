// keepquant.hip -- keep-quant grouped expert GEMMs on gfx950: GGUF Q4_K
// weight blocks against Q8_K-quantized activations with an integer MFMA core
// (PR #523 "What changed": the keep-quant expert GEMM family, Q8_K activation
// quantizer, super-block dot products with an integer core), carrying the
// BF16 path's epilogues: SiLU-mul after narrowing to bf16 (issue #3094 N1)
// and the routing weight on the f32 result before its one rounding (N2).
//
// Formats (GGUF): a Q4_K super-block holds 256 weights in 144 bytes: f16 d,
// f16 dmin, 12 bytes of six-bit scales sc_j and mins m_j for 8 sub-blocks of
// 32, then 128 bytes of 4-bit quants (byte b of 32-byte group i: value b of
// sub-block 2i in the low nibble, of sub-block 2i+1 in the high nibble);
// w = d * sc_j * q - dmin * m_j. A weight matrix [R, K] is R rows of K/256
// super-blocks. Q8_K activations (this library's layout, moe.h): int8 quants
// [R, K], f32 scales [R, K/256], int32 sums of 16 quants [R, K/16].
//
// Dot product of a weight row with an activation row, per super-block:
//   d_w d_x sum_j sc_j (sum_{l in j} q4_l q8_l) - dmin_w d_x sum_j m_j bsum_j
// Each sub-block's integer dot is one v_mfma_i32_16x16x32_i8 (16 activation
// rows x 16 weight rows x 32 k); the scale multiply and the mins term are
// integer; one f32 step per super-block.
#include "device_math.h"
#include "launch.h"

namespace moe {

typedef int i32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kQK = 256;        // values per super-block
constexpr int kQ4KBytes = 144;  // bytes per Q4_K super-block

extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);

// ---------------------------------------------------------------------------
// Q8_K quantizer: one wavefront per (row, super-block); lane l holds values
// 4l .. 4l+3. The entry of largest magnitude (the first one) gives
// iscale = -127 / max; q = min(127, round-half-even(iscale * x)); d = 1/iscale;
// an all-zero block gives d = 0 and q = 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_q8k_kernel(const uint16_t* __restrict__ x, int R,
                                                           int K, int8_t* __restrict__ qs,
                                                           float* __restrict__ dq,
                                                           int32_t* __restrict__ bsums) {
#pragma clang fp contract(off)
  const int nsb = K / kQK;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= R * nsb) return;  // whole wave leaves together
  const int lane = threadIdx.x & 63;
  const int r = wid / nsb, sb = wid - r * nsb;
  const size_t base = (size_t)r * K + (size_t)sb * kQK + lane * 4;
  const uint2 raw = *reinterpret_cast<const uint2*>(x + base);
  float v[4] = {bf16_to_f32(raw.x & 0xFFFFu), bf16_to_f32(raw.x >> 16),
                bf16_to_f32(raw.y & 0xFFFFu), bf16_to_f32(raw.y >> 16)};
  // largest magnitude of the block, then the first entry holding it
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) mine = max(mine, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  const uint32_t amax = __ockl_wfred_max_u32(mine);
  const uint64_t hit = __ballot(mine == amax);
  const int src = __ffsll((long long)hit) - 1;
  int first = 3;
#pragma unroll
  for (int i = 3; i >= 0; --i)
    if ((__float_as_uint(v[i]) & 0x7FFFFFFFu) == amax) first = i;
  float mx_l = v[0];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (first == i) mx_l = v[i];
  const float mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx_l), src));
  int q[4] = {0, 0, 0, 0};
  float d = 0.0f;
  if (amax != 0) {
    const float iscale = __fdiv_rn(-127.0f, mx);
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = min(127, (int)__builtin_rintf(iscale * v[i]));
    d = __fdiv_rn(1.0f, iscale);
  }
  const uint32_t packed = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) |
                          ((uint32_t)(q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24);
  *reinterpret_cast<uint32_t*>(qs + base) = packed;
  // sums of 16 quants: 4 lanes each
  int s = q[0] + q[1] + q[2] + q[3];
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  if ((lane & 3) == 0) bsums[(size_t)r * (K / 16) + sb * 16 + (lane >> 2)] = s;
  if (lane == 0) dq[(size_t)r * nsb + sb] = d;
}

// ---------------------------------------------------------------------------
// Grouped keep-quant GEMM, few rows per expert (decode): one workgroup = one
// 16-row tile of one expert x 16*NFO output columns (gate-up: each group of
// 16 gate rows with the 16 matching up rows); its KS waves split the
// super-blocks and add their partial f32 tiles in LDS in a fixed order. The
// activation side of a super-block (A operands, scales, sums) is loaded once
// per wave and used by all its weight fragments.
// ---------------------------------------------------------------------------
struct KqArgs {
  const int8_t* xq;        // activation quants [a_rows, kdim]
  const float* xd;         // activation scales [a_rows, kdim / 256]
  const int32_t* xs;       // activation sums of 16 [a_rows, kdim / 16]
  int a_rows;
  const int32_t* sorted;   // sorted pair ids, or null
  int gather_k;            // >0: activation row = sorted[q] / gather_k; 0: row q
  const uint8_t* W;        // Q4_K weights [E, b_rows, kdim / 256, 144]
  int b_rows;              // 2I (gate-up) or H (down)
  const int32_t* offsets;  // [E+1] or null
  int E, P, kdim, n_out;
  uint16_t* out;
  const float* pair_w;
  int slots, nblk;
};

enum { KQ_GATEUP = 0, KQ_DOWN = 1 };

// the same tile lookup as the BF16 GEMMs: slot -> (expert, first row, rows)
__device__ __forceinline__ bool kq_find_tile(const KqArgs& g, int slot, int& e, int& row0,
                                             int& rows) {
  constexpr int BM = 16;
  if (g.offsets == nullptr) {
    const int r0 = slot * BM;
    if (r0 >= g.P) return false;
    e = 0;
    row0 = r0;
    rows = min(BM, g.P - r0);
    return true;
  }
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int base = 0; base < g.E; base += 64) {
    const int ex = base + lane;
    int o0 = 0, cnt = 0;
    if (ex < g.E) {
      o0 = min(max(g.offsets[ex], 0), g.P);
      const int o1 = min(max(g.offsets[ex + 1], 0), g.P);
      cnt = max(0, o1 - o0);
    }
    const int nt = (cnt + BM - 1) / BM;
    int incl = nt;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(incl, m);
      if (lane >= m) incl += o;
    }
    const int first = before + incl - nt;
    const uint64_t hit = __ballot(nt > 0 && slot >= first && slot < first + nt);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      e = __builtin_amdgcn_readlane(ex, src);
      const int f = __builtin_amdgcn_readlane(first, src);
      const int oo = __builtin_amdgcn_readlane(o0, src);
      const int cc = __builtin_amdgcn_readlane(cnt, src);
      row0 = oo + (slot - f) * BM;
      rows = min(BM, cc - (slot - f) * BM);
      return true;
    }
    before += __builtin_amdgcn_readlane(incl, 63);
  }
  return false;
}

__device__ __forceinline__ uint32_t kq_rsrc_size(size_t bytes) {
  return bytes < 0x7FFFFFFFu ? (uint32_t)bytes : 0x7FFFFFFFu;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t kq_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)kq_rsrc_size(bytes), 0x00020000);
}

constexpr uint32_t kqOob = 0x80000000u;

template <int EPI, int KS, int NFO>
__global__ __launch_bounds__(64 * KS) void kq_stream_kernel(KqArgs g) {
#pragma clang fp contract(off)
  // weight fragments of 16 rows: NFO column groups, each gate (and up)
  constexpr int NB = (EPI == KQ_GATEUP) ? 2 * NFO : NFO;
  __shared__ float red[KS][NB][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = blockIdx.x / g.nblk;
  const int nb = blockIdx.x - slot * g.nblk;
  int e, row0, rows;
  if (!kq_find_tile(g, slot, e, row0, rows)) return;  // uniform over the workgroup
  const int col0 = nb * 16 * NFO;
  const int r16 = lane & 15;   // A row / B column of this lane's MFMA operands
  const int kc = lane >> 4;    // 8-value k chunk of a 32-value sub-block
  const int nsb = g.kdim / kQK;

  // activation row of this lane's A operand, and of its 4 C rows
  auto act_row = [&](int rr) -> int {
    if (rr >= rows) return -1;
    const int q = row0 + rr;
    int a = q;
    if (g.sorted != nullptr && g.gather_k > 0) {
      const int p = g.sorted[q];
      a = (p < 0) ? -1 : p / g.gather_k;
    }
    return (a >= 0 && a < g.a_rows) ? a : -1;
  };
  const int arow = act_row(r16);
  int crow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) crow[i] = act_row(kc * 4 + i);

  const size_t a_rows = (size_t)g.a_rows;
  const __amdgpu_buffer_rsrc_t rq = kq_rsrc(g.xq, a_rows * g.kdim);
  const __amdgpu_buffer_rsrc_t rd = kq_rsrc(g.xd, a_rows * nsb * 4);
  const __amdgpu_buffer_rsrc_t rs = kq_rsrc(g.xs, a_rows * (g.kdim / 16) * 4);
  const size_t row_bytes = (size_t)nsb * kQ4KBytes;
  const __amdgpu_buffer_rsrc_t rw =
      kq_rsrc(g.W + (size_t)e * g.b_rows * row_bytes, (size_t)g.b_rows * row_bytes);

  // byte offsets (super-block 0) of this lane's weight rows: fragment f is
  // column group f / 2 (gate-up: f even gate, f odd up) or f (down)
  uint32_t wrow[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f) {
    const int fo = (EPI == KQ_GATEUP) ? (f >> 1) : f;
    const int c = col0 + fo * 16 + r16;
    const int wr = (EPI == KQ_GATEUP && (f & 1)) ? g.n_out + c : c;
    wrow[f] = (c < g.n_out) ? (uint32_t)(wr * row_bytes) : kqOob;
  }
  const uint32_t aq_off = (arow >= 0) ? (uint32_t)((size_t)arow * g.kdim) + kc * 8 : kqOob;

  float acc[NB][4];
#pragma unroll
  for (int f = 0; f < NB; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[f][i] = 0.0f;

  // this wave's super-blocks
  const int per = (nsb + KS - 1) / KS;
  const int sb0 = min(nsb, wave * per), sb1 = min(nsb, sb0 + per);
  for (int sb = sb0; sb < sb1; ++sb) {
    // activation side, shared by every fragment: A operands of the 8
    // sub-blocks, sub-block sums, and the scales of the 4 C rows
    long aop[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t ao = (aq_off == kqOob) ? kqOob : aq_off + sb * kQK + j * 32;
      aop[j] = (long)__builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rq, ao, 0, 0));
    }
    // A operands of the mins term: sums of the 32 quants of sub-blocks kc
    // and kc + 4 of activation row r16
    float bsa[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t so =
          (arow < 0) ? kqOob : (uint32_t)(arow * (g.kdim / 16) + sb * 16 + 2 * (kc + 4 * h)) * 4;
      const uint2 s2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, so, 0, 0));
      bsa[h] = (float)((int)s2.x + (int)s2.y);
    }
    float dx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ro = (crow[i] >= 0) ? (uint32_t)(crow[i] * nsb + sb) * 4 : kqOob;
      dx[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, ro, 0, 0));
    }
    // every fragment's weight loads first (headers: f16 d, f16 dmin, 12
    // bytes of six-bit scales and mins; then the quants), so that the
    // whole super-block is in flight before the first MFMA
    const uint32_t sboff = (uint32_t)sb * kQ4KBytes;
    i32x4v hdrs[NB];
    uint2 w8s[NB][4];
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const uint32_t ho = (wrow[f] == kqOob) ? kqOob : wrow[f] + sboff;
      hdrs[f] = __builtin_bit_cast(i32x4v, __builtin_amdgcn_raw_buffer_load_b128(rw, ho, 0, 0));
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t qo = (ho == kqOob) ? kqOob : ho + 16 + p * 32 + kc * 8;
        w8s[f][p] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rw, qo, 0, 0));
      }
    }
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      // one fragment at a time: keeps the MFMA results of only one
      // fragment live
      __builtin_amdgcn_sched_barrier(0);
      const i32x4v hdr = hdrs[f];
      const uint2* w8 = w8s[f];
      const float dw = (float)__builtin_bit_cast(_Float16, (uint16_t)(hdr.x & 0xFFFF));
      const float dmw = (float)__builtin_bit_cast(_Float16, (uint16_t)((uint32_t)hdr.x >> 16));
      // scales of the 8 sub-blocks: bytes 0-3 (low 6 bits) give sc_0..3;
      // bytes 8-11 (low nibble) with the top 2 bits of bytes 0-3 give sc_4..7
      const uint32_t b03 = (uint32_t)hdr.y, b47 = (uint32_t)hdr.z, b811 = (uint32_t)hdr.w;
      int sc[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = (b03 >> (8 * j)) & 63;
        sc[j + 4] = ((b811 >> (8 * j)) & 0xF) | (((b03 >> (8 * j + 6)) & 3) << 4);
      }
      // B operands of the mins term: m_kc and m_kc+4 of this lane's column
      // (bytes 4-7 low 6 bits; bytes 8-11 high nibble with the top 2 bits
      // of bytes 4-7)
      const uint32_t sh = 8u * (uint32_t)kc;
      const float mnb0 = (float)((b47 >> sh) & 63);
      const float mnb1 = (float)(((b811 >> (sh + 4)) & 0xF) | (((b47 >> (sh + 6)) & 3) << 4));
      // integer sub-block dots, scaled by sc_j (this lane's column)
      int sumi[4] = {0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int j = 2 * p + half;
          const uint32_t lo = half ? ((w8[p].x >> 4) & 0x0F0F0F0Fu) : (w8[p].x & 0x0F0F0F0Fu);
          const uint32_t hi = half ? ((w8[p].y >> 4) & 0x0F0F0F0Fu) : (w8[p].y & 0x0F0F0F0Fu);
          const long bop = (long)(((uint64_t)hi << 32) | lo);
          const i32x4v z = {0, 0, 0, 0};
          const i32x4v dot = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[j], bop, z, 0, 0, 0);
          // |dot| <= 32 * 15 * 127 and sc_j <= 63: 24-bit products suffice
          sumi[0] += __mul24(sc[j], dot.x);
          sumi[1] += __mul24(sc[j], dot.y);
          sumi[2] += __mul24(sc[j], dot.z);
          sumi[3] += __mul24(sc[j], dot.w);
        }
      }
      // mins term sum_j m_j bsum_j of the 4 C rows: integers below 2^21,
      // exact in f32
      const f32x4v zf = {0.0f, 0.0f, 0.0f, 0.0f};
      f32x4v summ = __builtin_amdgcn_mfma_f32_16x16x4f32(bsa[0], mnb0, zf, 0, 0, 0);
      summ = __builtin_amdgcn_mfma_f32_16x16x4f32(bsa[1], mnb1, summ, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dall = dw * dx[i];
        const float dmn = dmw * dx[i];
        const float t1 = dall * (float)sumi[i];
        const float t2 = dmn * summ[i];
        acc[f][i] = acc[f][i] + (t1 - t2);
      }
    }
  }

#pragma unroll
  for (int f = 0; f < NB; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][f][i][lane] = acc[f][i];
  __syncthreads();
  // C layout: element i of lane l is row (l/16)*4 + i, column l%16; wave w
  // finishes the elements i = w, w + KS, ...: fixed-order sum over waves
  for (int i = wave; i < 4; i += KS) {
    const int rr = kc * 4 + i;
    if (rr >= rows) continue;
    const int q = row0 + rr;
#pragma unroll
    for (int fo = 0; fo < NFO; ++fo) {
      const int c = col0 + fo * 16 + r16;
      constexpr int PER = (EPI == KQ_GATEUP) ? 2 : 1;
      float sum[PER];
#pragma unroll
      for (int h = 0; h < PER; ++h) {
        float s = red[0][fo * PER + h][i][lane];
#pragma unroll
        for (int w = 1; w < KS; ++w) s = s + red[w][fo * PER + h][i][lane];
        sum[h] = s;
      }
      if (c >= g.n_out) continue;
      if (EPI == KQ_GATEUP) {
        const float gb = round_bf16(sum[0]);  // N1
        const float ub = round_bf16(sum[PER - 1]);
        g.out[(size_t)q * g.n_out + c] = (uint16_t)f32_to_bf16(silu_cw(gb) * ub);
      } else {
        const int p = (g.sorted != nullptr) ? g.sorted[q] : q;
        if (p < 0 || p >= g.P) continue;
        float y = sum[0];
        if (g.pair_w != nullptr) y = y * g.pair_w[p];  // N2
        g.out[(size_t)p * g.n_out + c] = (uint16_t)f32_to_bf16(y);
      }
    }
  }
}

static inline int kq_slots(int P, int E, bool grouped) {
  const int full = (P + 15) / 16;
  return grouped ? full + (E < P ? E : P) : full;
}

hipError_t launch_quantize_q8k(const uint16_t* x, int R, int K, int8_t* qs, float* d,
                               int32_t* bsums, hipStream_t s) {
  const int waves = R * (K / kQK);
  hipLaunchKernelGGL(quantize_q8k_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, x, R, K, qs, d,
                     bsums);
  return hipGetLastError();
}

template <int EPI, int KS, int NFO>
static hipError_t kq_launch_shape(KqArgs g, hipStream_t s) {
  g.nblk = (g.n_out + 16 * NFO - 1) / (16 * NFO);
  g.slots = kq_slots(g.P, g.E, g.offsets != nullptr);
  const unsigned grid = (unsigned)((long long)g.slots * g.nblk);
  void* args[] = {&g};
  return timed_launch(reinterpret_cast<const void*>(kq_stream_kernel<EPI, KS, NFO>), dim3(grid),
                      dim3(64 * KS), args, s);
}

// k split over as many waves as there are super-blocks (at most 4); 64
// output columns per workgroup
template <int EPI>
static hipError_t kq_launch(KqArgs g, hipStream_t s) {
  const int nsb = g.kdim / kQK;
  if (nsb >= 4) return kq_launch_shape<EPI, 4, 4>(g, s);
  if (nsb == 3) return kq_launch_shape<EPI, 3, 4>(g, s);
  if (nsb == 2) return kq_launch_shape<EPI, 2, 4>(g, s);
  return kq_launch_shape<EPI, 1, 4>(g, s);
}

hipError_t launch_kq_gateup_silu(const int8_t* xq, const float* xd, const int32_t* xs, int T, int H,
                                 const uint8_t* w_gu, int E, int I, const int32_t* sorted,
                                 const int32_t* offsets, int K, uint16_t* act, hipStream_t s) {
  KqArgs g{};
  g.xq = xq; g.xd = xd; g.xs = xs; g.a_rows = T;
  g.sorted = sorted; g.gather_k = K;
  g.W = w_gu; g.b_rows = 2 * I;
  g.offsets = offsets; g.E = E; g.P = T * K; g.kdim = H; g.n_out = I;
  g.out = act;
  return kq_launch<KQ_GATEUP>(g, s);
}

hipError_t launch_kq_down(const int8_t* aq, const float* ad, const int32_t* as, int P, int I,
                          const uint8_t* w_d, int E, int H, const int32_t* sorted,
                          const int32_t* offsets, const float* pair_w, uint16_t* out,
                          hipStream_t s) {
  KqArgs g{};
  g.xq = aq; g.xd = ad; g.xs = as; g.a_rows = P;
  g.sorted = sorted; g.gather_k = 0;
  g.W = w_d; g.b_rows = H;
  g.offsets = offsets; g.E = E; g.P = P; g.kdim = I; g.n_out = H;
  g.out = out; g.pair_w = pair_w;
  return kq_launch<KQ_DOWN>(g, s);
}

}  // namespace moe
