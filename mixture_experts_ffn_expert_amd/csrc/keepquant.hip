// keepquant.hip -- keep-quant grouped expert GEMMs on gfx950: GGUF weight
// blocks (Q4_K, Q5_K, Q6_K, Q8_0) against activations quantized on the fly
// (Q8_K for the K-quants, Q8_0 for Q8_0 weights) with an integer MFMA core
// (PR #523 "What changed": the keep-quant expert GEMM family, the Q8_0 and
// Q8_K activation quantizers, block dot products with an integer core),
// carrying the BF16 path's epilogues: SiLU-mul after narrowing to bf16 (issue
// #3094 N1) and the routing weight on the f32 result before its one rounding
// (N2).
//
// Formats (GGUF), per block:
//   Q4_K, 256 values in 144 B: f16 d, f16 dmin, 12 B of six-bit scales sc_j
//     and mins m_j (8 sub-blocks of 32), 128 B of nibbles (byte b of 32-byte
//     group i: value b of sub-block 2i low, of sub-block 2i+1 high);
//     w = d sc_j q - dmin m_j.
//   Q5_K, 256 values in 176 B: as Q4_K with 32 B of high bits qh between the
//     scales and the nibbles; value b of sub-block j adds 16 * bit j of qh[b].
//   Q6_K, 256 values in 210 B: 128 B of low nibbles ql, 64 B of 2-bit highs
//     qh, 16 int8 scales (sub-blocks of 16), f16 d. For half h, c < 4, l < 32
//     the value 128h + 32c + l is the low (c < 2) or high (c >= 2) nibble of
//     ql[64h + 32(c%2) + l] with bits 2c, 2c+1 of qh[32h + l] above it, less
//     32; w = d sc_{v/16} q.
//   Q8_0, 32 values in 34 B: f16 d, 32 int8 quants; w = d q.
// Activations (this library's layouts, moe.h): Q8_K int8 [R, K], f32 scales
// [R, K/256], int32 sums of 16 [R, K/16]; Q8_0 int8 [R, K], f16 scales
// [R, K/32].
//
// Dot product of a weight row with an activation row per unit of 256 values
// (one K-quant super-block, eight Q8_0 blocks):
//   Q4_K, Q5_K: d_w d_x sum_j sc_j dot_j - dmin_w d_x sum_j m_j bsum32_j
//   Q6_K:       d_w d_x (sum_j sc_j dot_j - 32 sum_j sc_j bsum16_j)
//   Q8_0:       sum_b d_w,b d_x,b dot_b
// where dot_j is the integer dot of the codes (Q6_K: the unsigned 6-bit
// codes). One v_mfma_i32_16x16x32_i8 (16 activation rows x 16 weight rows x
// 32 k) gives the dots of a 32-value group; Q6_K's two 16-value sub-blocks of
// a group come from two MFMAs whose activation operand keeps one k half
// each. The sc_j dot_j sums are integer (24-bit products); the mins and
// offset sums are exact f32 MFMAs (16x16x4) over the activation's sub-block
// sums; then one f32 step per unit (per block for Q8_0).
#include "device_math.h"
#include "launch.h"

namespace moe {

typedef int i32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x3v __attribute__((ext_vector_type(3)));

constexpr int kQK = 256;  // values per super-block (and per unit of eight Q8_0 blocks)

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
// Q8_0 quantizer: four lanes per block of 32 (8 values each); amax over the
// block, d = amax / 127, id = 1/d (0 when d = 0), q = round-half-away(x * id),
// d stored as f16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const uint16_t* __restrict__ x,
                                                            long long nblk,
                                                            int8_t* __restrict__ qs,
                                                            uint16_t* __restrict__ dq) {
#pragma clang fp contract(off)
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long blk = t >> 2;
  // 4 lanes of a block are consecutive; a wave holds whole blocks, so the
  // shuffles below stay inside active lanes
  if (blk >= nblk) return;
  const int part = (int)(t & 3);
  const size_t base = (size_t)blk * 32 + part * 8;
  const uint4 raw = *reinterpret_cast<const uint4*>(x + base);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const float d = __fdiv_rn(amax, 127.0f);
  const float id = (d != 0.0f) ? __fdiv_rn(1.0f, d) : 0.0f;
  uint32_t packed[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = (int)__builtin_roundf(v[i] * id);  // half away from zero
    packed[i >> 2] |= (uint32_t)(q & 0xFF) << (8 * (i & 3));
  }
  *reinterpret_cast<uint2*>(qs + base) = make_uint2(packed[0], packed[1]);
  if (part == 0) dq[blk] = __builtin_bit_cast(uint16_t, (_Float16)d);
}

// ---------------------------------------------------------------------------
// Grouped keep-quant GEMM, few rows per expert (decode): one workgroup = one
// 16-row tile of one expert x 16*NFO output columns (gate-up: each group of
// 16 gate rows with the 16 matching up rows); its KS waves split the units of
// 256 values and add their partial f32 tiles in LDS in a fixed order. The
// activation side of a unit is loaded once per wave and used by all its
// weight fragments; every fragment's weight loads are issued before the
// first MFMA of the unit.
// ---------------------------------------------------------------------------
enum { KQ_Q8_0 = 8, KQ_Q4_K = 12, KQ_Q5_K = 13, KQ_Q6_K = 14 };

// bytes per unit of 256 values
template <int FMT>
constexpr int kq_unit_bytes() {
  return FMT == KQ_Q4_K ? 144 : FMT == KQ_Q5_K ? 176 : FMT == KQ_Q6_K ? 210 : 272;
}

struct KqArgs {
  const int8_t* xq;        // activation quants [a_rows, kdim]
  const void* xd;          // activation scales: f32 [a_rows, kdim/256] or f16 [a_rows, kdim/32]
  const int32_t* xs;       // activation sums of 16 [a_rows, kdim / 16] (Q8_K only)
  int a_rows;
  const int32_t* sorted;   // sorted pair ids, or null
  int gather_k;            // >0: activation row = sorted[q] / gather_k; 0: row q
  const uint8_t* W;        // weight blocks [E, b_rows, kdim / 256 units]
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

// 8 bytes at a 2-aligned offset: one dword-aligned 12-byte load, realigned
// (the load starts at most 2 bytes before off and ends 4 bytes after off+7)
__device__ __forceinline__ uint2 kq_load8_a2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const uint32_t sh = off & 3u;
  const u32x3v w = __builtin_bit_cast(u32x3v, __builtin_amdgcn_raw_buffer_load_b96(r, off - sh, 0, 0));
  return make_uint2(__builtin_amdgcn_alignbyte(w.y, w.x, sh), __builtin_amdgcn_alignbyte(w.z, w.y, sh));
}

__device__ __forceinline__ uint2 kq_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// Coalesced operand loads. In the order of a v_mfma_i32_16x16x32_i8 operand
// lane l holds row l % 16, 8-byte chunk l / 16 of a 32-value group, so a
// load in that order has its 64 lanes read 64 separate 8-byte pieces. The
// code bytes (activation codes; Q4_K / Q5_K nibbles and high bits) are
// loaded with four consecutive lanes reading one row's 32 bytes (row l / 4,
// chunk l % 4) instead, and this permutation (psrc: byte index of the
// source lane) puts each lane's 8 bytes in MFMA order.
__device__ __forceinline__ uint2 kq_perm8(uint2 v, int psrc) {
  return make_uint2((uint32_t)__builtin_amdgcn_ds_bpermute(psrc, (int)v.x),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(psrc, (int)v.y));
}

__device__ __forceinline__ long kq_pair(uint32_t lo, uint32_t hi) {
  return (long)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float kq_f16(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

// Weight registers of one 16-row fragment for one unit, per format.
template <int FMT>
struct KqW;
template <>
struct KqW<KQ_Q4_K> {
  i32x4v hdr;
  uint2 qs[4];
};
template <>
struct KqW<KQ_Q5_K> {
  i32x4v hdr;
  uint2 qh;
  uint2 qs[4];
};
template <>
struct KqW<KQ_Q6_K> {
  uint2 ql[4];   // (half h, column pair c2): index 2h + c2
  uint2 qh[2];
  i32x4v sc;     // 16 scale bytes, dword-aligned copy of offsets 192 - sh ..
  uint32_t sc_tail, dbits, sh;
};
template <>
struct KqW<KQ_Q8_0> {
  uint2 q[8];
  uint32_t d2;  // f16 scales of blocks 2 kc (low half) and 2 kc + 1 (high half)
};

// Loads the unit at byte offset `base` (kqOob-based offsets stay out of
// range) of this lane's weight row; lane chunk kc of every 32-value group.
// The code bytes come coalesced from the unit at base_c of row l / 4 (chunk
// kcc = l % 4) and are permuted into MFMA order; headers, scales and the
// Q8_0 block scales are read for this lane's own row.
template <int FMT, bool CO>
__device__ __forceinline__ void kq_wload(KqW<FMT>& w, __amdgpu_buffer_rsrc_t r, uint32_t base,
                                         int kc, uint32_t base_c, int kcc, int psrc) {
  if constexpr (!CO) {  // code bytes in MFMA order, straight from this lane's row
    base_c = base;
    kcc = kc;
  }
  auto perm = [&](uint2 v) -> uint2 {
    if constexpr (CO) return kq_perm8(v, psrc);
    return v;
  };
  if constexpr (FMT == KQ_Q4_K) {
    w.hdr = __builtin_bit_cast(i32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, base, 0, 0));
#pragma unroll
    for (int p = 0; p < 4; ++p) w.qs[p] = kq_load8(r, base_c + 16 + p * 32 + kcc * 8);
#pragma unroll
    for (int p = 0; p < 4; ++p) w.qs[p] = perm(w.qs[p]);
  } else if constexpr (FMT == KQ_Q5_K) {
    w.hdr = __builtin_bit_cast(i32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, base, 0, 0));
    w.qh = kq_load8(r, base_c + 16 + kcc * 8);
#pragma unroll
    for (int p = 0; p < 4; ++p) w.qs[p] = kq_load8(r, base_c + 48 + p * 32 + kcc * 8);
    w.qh = perm(w.qh);
#pragma unroll
    for (int p = 0; p < 4; ++p) w.qs[p] = perm(w.qs[p]);
  } else if constexpr (FMT == KQ_Q6_K) {
    // 210-byte blocks: base is 2-aligned; every load stays in [base - 2,
    // base + 210)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
        w.ql[2 * h + c2] = kq_load8_a2(r, base_c + 64 * h + 32 * c2 + kcc * 8);
#pragma unroll
    for (int h = 0; h < 2; ++h) w.qh[h] = kq_load8_a2(r, base_c + 128 + 32 * h + kcc * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) w.ql[i] = perm(w.ql[i]);
#pragma unroll
    for (int h = 0; h < 2; ++h) w.qh[h] = perm(w.qh[h]);
    w.sh = base & 3u;
    w.sc = __builtin_bit_cast(i32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, base + 192 - w.sh, 0, 0));
    w.sc_tail = __builtin_amdgcn_raw_buffer_load_b16(r, base + 206, 0, 0);
    w.dbits = __builtin_amdgcn_raw_buffer_load_b16(r, base + 208, 0, 0);
  } else {
    // eight 34-byte blocks; base is 4-aligned (rows of 272-byte units), so
    // the quants of even blocks sit 2 bytes past a dword boundary
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint32_t qo = base_c + 34 * b + 2 + kcc * 8;
      w.q[b] = (b & 1) ? kq_load8(r, qo) : kq_load8_a2(r, qo);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) w.q[b] = perm(w.q[b]);
    // the four lanes of a row share its 8 scales: lane chunk kc loads two
    // of them, the others come by lane exchange (kq_frag)
    const uint32_t dl = __builtin_amdgcn_raw_buffer_load_b16(r, base + 68 * kc, 0, 0);
    const uint32_t dh = __builtin_amdgcn_raw_buffer_load_b16(r, base + 68 * kc + 34, 0, 0);
    w.d2 = (dl & 0xFFFFu) | (dh << 16);
  }
}

// Activation registers of one unit, per activation format.
template <int FMT>
struct KqA {
  long aop[8];      // A operands of the 8 groups of 32 (this lane's row r16, chunk kc)
  float bsa[4];     // A operands of the mins / offset MFMAs
  float dx[4][8];   // scales of the 4 C rows (K-quants: [i][0]; Q8_0: per block)
};

// The activation codes come coalesced from row arow_c (chunk kcc) and are
// permuted into MFMA order; scales and sums are read in MFMA order.
template <int FMT, bool CO>
__device__ __forceinline__ void kq_aload(KqA<FMT>& a, const KqArgs& g,
                                         __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rd,
                                         __amdgpu_buffer_rsrc_t rs, int arow, const int* crow,
                                         int u, int kc, int arow_c, int kcc, int psrc) {
  if constexpr (!CO) {
    arow_c = arow;
    kcc = kc;
  }
  const uint32_t aq =
      (arow_c >= 0) ? (uint32_t)arow_c * (uint32_t)g.kdim + u * kQK + kcc * 8 : kqOob;
  uint2 ac[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ac[j] = kq_load8(rq, aq + j * 32);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    a.aop[j] = (long)__builtin_bit_cast(uint64_t, CO ? kq_perm8(ac[j], psrc) : ac[j]);
  const int nsb = g.kdim / kQK;
  if constexpr (FMT == KQ_Q8_0) {
    // 8 f16 scales per row and unit: one 16-byte load per C row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = (crow[i] >= 0) ? ((uint32_t)crow[i] * (g.kdim / 32) + u * 8) * 2 : kqOob;
      const i32x4v h = __builtin_bit_cast(i32x4v, __builtin_amdgcn_raw_buffer_load_b128(rd, o, 0, 0));
      const uint32_t hw[4] = {(uint32_t)h.x, (uint32_t)h.y, (uint32_t)h.z, (uint32_t)h.w};
#pragma unroll
      for (int b = 0; b < 8; ++b) a.dx[i][b] = kq_f16(hw[b >> 1] >> (16 * (b & 1)));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = (crow[i] >= 0) ? ((uint32_t)crow[i] * nsb + u) * 4 : kqOob;
      a.dx[i][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, o, 0, 0));
    }
    const uint32_t so = (arow >= 0) ? ((uint32_t)arow * (g.kdim / 16) + u * 16) * 4 : kqOob;
    if constexpr (FMT == KQ_Q6_K) {
      // sums of 16 of sub-blocks 4m + kc
#pragma unroll
      for (int m = 0; m < 4; ++m)
        a.bsa[m] = (float)(int)__builtin_amdgcn_raw_buffer_load_b32(rs, so + (4 * m + kc) * 4, 0, 0);
    } else {
      // sums of 32 of sub-blocks kc and kc + 4
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint2 s2 = kq_load8(rs, so + 2 * (kc + 4 * h) * 4);
        a.bsa[h] = (float)((int)s2.x + (int)s2.y);
      }
    }
  }
}

// Scales and mins of a Q4_K / Q5_K header for this lane's column.
__device__ __forceinline__ void kq_scales_k4(const i32x4v hdr, int kc, int* sc, float& mnb0,
                                             float& mnb1) {
  // bytes 0-3 (low 6 bits) give sc_0..3; bytes 8-11 (low nibble) with the
  // top 2 bits of bytes 0-3 give sc_4..7
  const uint32_t b03 = (uint32_t)hdr.y, b47 = (uint32_t)hdr.z, b811 = (uint32_t)hdr.w;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sc[j] = (b03 >> (8 * j)) & 63;
    sc[j + 4] = ((b811 >> (8 * j)) & 0xF) | (((b03 >> (8 * j + 6)) & 3) << 4);
  }
  // B operands of the mins MFMAs: m_kc and m_kc+4 (bytes 4-7 low 6 bits;
  // bytes 8-11 high nibble with the top 2 bits of bytes 4-7)
  const uint32_t sh = 8u * (uint32_t)kc;
  mnb0 = (float)((b47 >> sh) & 63);
  mnb1 = (float)(((b811 >> (sh + 4)) & 0xF) | (((b47 >> (sh + 6)) & 3) << 4));
}

// One fragment's contribution for one unit: acc[i] (C row kc*4 + i, this
// lane's column) += the unit's dot product.
template <int FMT>
__device__ __forceinline__ void kq_frag(float* acc, const KqW<FMT>& w, const KqA<FMT>& a,
                                        const long* alo, const long* ahi, int kc) {
#pragma clang fp contract(off)
  const i32x4v z = {0, 0, 0, 0};
  const f32x4v zf = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr uint32_t M4 = 0x0F0F0F0Fu;
  if constexpr (FMT == KQ_Q4_K || FMT == KQ_Q5_K) {
    const float dw = kq_f16((uint32_t)w.hdr.x);
    const float dmw = kq_f16((uint32_t)w.hdr.x >> 16);
    int sc[8];
    float mnb0, mnb1;
    kq_scales_k4(w.hdr, kc, sc, mnb0, mnb1);
    int sumi[4] = {0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int j = 2 * p + half;
        uint32_t lo = half ? ((w.qs[p].x >> 4) & M4) : (w.qs[p].x & M4);
        uint32_t hi = half ? ((w.qs[p].y >> 4) & M4) : (w.qs[p].y & M4);
        if constexpr (FMT == KQ_Q5_K) {
          // bit j of each qh byte -> bit 4 of the code
          lo |= ((w.qh.x >> j) & 0x01010101u) << 4;
          hi |= ((w.qh.y >> j) & 0x01010101u) << 4;
        }
        const i32x4v dot = __builtin_amdgcn_mfma_i32_16x16x32_i8(a.aop[j], kq_pair(lo, hi), z, 0, 0, 0);
        // |dot| <= 32 * 31 * 127 and sc_j <= 63: 24-bit operands
        sumi[0] += __mul24(sc[j], dot.x);
        sumi[1] += __mul24(sc[j], dot.y);
        sumi[2] += __mul24(sc[j], dot.z);
        sumi[3] += __mul24(sc[j], dot.w);
      }
    }
    // mins term sum_j m_j bsum32_j of the 4 C rows: integers below 2^22
    f32x4v summ = __builtin_amdgcn_mfma_f32_16x16x4f32(a.bsa[0], mnb0, zf, 0, 0, 0);
    summ = __builtin_amdgcn_mfma_f32_16x16x4f32(a.bsa[1], mnb1, summ, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float dall = dw * a.dx[i][0];
      const float dmn = dmw * a.dx[i][0];
      const float t1 = dall * (float)sumi[i];
      const float t2 = dmn * summ[i];
      acc[i] = acc[i] + (t1 - t2);
    }
  } else if constexpr (FMT == KQ_Q6_K) {
    const float dw = kq_f16(w.dbits);
    // the 16 scale bytes, realigned: s[m] holds scales 4m .. 4m+3
    const uint32_t s[4] = {
        __builtin_amdgcn_alignbyte((uint32_t)w.sc.y, (uint32_t)w.sc.x, w.sh),
        __builtin_amdgcn_alignbyte((uint32_t)w.sc.z, (uint32_t)w.sc.y, w.sh),
        __builtin_amdgcn_alignbyte((uint32_t)w.sc.w, (uint32_t)w.sc.z, w.sh),
        __builtin_amdgcn_alignbyte(w.sc_tail, (uint32_t)w.sc.w, w.sh)};
    int sumi[4] = {0, 0, 0, 0};
#pragma unroll
    for (int grp = 0; grp < 8; ++grp) {
      const int h = grp >> 2, c = grp & 3;
      const uint2 ql = w.ql[2 * h + (c & 1)];
      const uint2 qh = w.qh[h];
      const uint32_t lo = ((c < 2 ? ql.x : (ql.x >> 4)) & M4) | (((qh.x >> (2 * c)) & 0x03030303u) << 4);
      const uint32_t hi = ((c < 2 ? ql.y : (ql.y >> 4)) & M4) | (((qh.y >> (2 * c)) & 0x03030303u) << 4);
      const long bop = kq_pair(lo, hi);
      // sub-blocks 2 grp (k 0-15 of the group) and 2 grp + 1 (k 16-31)
      const i32x4v da = __builtin_amdgcn_mfma_i32_16x16x32_i8(alo[grp], bop, z, 0, 0, 0);
      const i32x4v db = __builtin_amdgcn_mfma_i32_16x16x32_i8(ahi[grp], bop, z, 0, 0, 0);
      const int j = 2 * grp;
      const int sa = (int)(s[j >> 2] << (24 - 8 * (j & 3))) >> 24;
      const int sb = (int)(s[(j + 1) >> 2] << (24 - 8 * ((j + 1) & 3))) >> 24;
      // |dot| <= 16 * 63 * 127, |sc| <= 128: 24-bit operands
      sumi[0] += __mul24(sa, da.x) + __mul24(sb, db.x);
      sumi[1] += __mul24(sa, da.y) + __mul24(sb, db.y);
      sumi[2] += __mul24(sa, da.z) + __mul24(sb, db.z);
      sumi[3] += __mul24(sa, da.w) + __mul24(sb, db.w);
    }
    // offset term sum_j sc_j bsum16_j: integers below 2^23, exact in f32
    f32x4v so = zf;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float scb = (float)((int)(s[m] << (24 - 8 * kc)) >> 24);
      so = __builtin_amdgcn_mfma_f32_16x16x4f32(a.bsa[m], scb, so, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int total = sumi[i] - 32 * (int)so[i];
      acc[i] = acc[i] + (dw * a.dx[i][0]) * (float)total;
    }
  } else {
    // scales of blocks 2m, 2m + 1 from the lane of chunk m of this row
    const int r16 = threadIdx.x & 15;
    uint32_t dsc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) dsc[m] = (uint32_t)__shfl((int)w.d2, r16 + 16 * m);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const i32x4v dot =
          __builtin_amdgcn_mfma_i32_16x16x32_i8(a.aop[b], kq_pair(w.q[b].x, w.q[b].y), z, 0, 0, 0);
      const float dw = kq_f16(dsc[b >> 1] >> (16 * (b & 1)));
      acc[0] = acc[0] + (dw * a.dx[0][b]) * (float)dot.x;
      acc[1] = acc[1] + (dw * a.dx[1][b]) * (float)dot.y;
      acc[2] = acc[2] + (dw * a.dx[2][b]) * (float)dot.z;
      acc[3] = acc[3] + (dw * a.dx[3][b]) * (float)dot.w;
    }
  }
}

template <int EPI, int FMT, int KS, int NFO>
__global__ __launch_bounds__(64 * KS) void kq_stream_kernel(KqArgs g) {
#pragma clang fp contract(off)
  // weight fragments of 16 rows: NFO column groups, each gate (and up)
  constexpr int NB = (EPI == KQ_GATEUP) ? 2 * NFO : NFO;
  constexpr int UB = kq_unit_bytes<FMT>();
  __shared__ float red[KS][NB][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = blockIdx.x / g.nblk;
  const int nb = blockIdx.x - slot * g.nblk;
  int e, row0, rows;
  if (!kq_find_tile(g, slot, e, row0, rows)) return;  // uniform over the workgroup
  const int col0 = nb * 16 * NFO;
  const int r16 = lane & 15;   // A row / B column of this lane's MFMA operands
  const int kc = lane >> 4;    // 8-value k chunk of a 32-value group
  // coalesced loads (gate-up): row lane / 4, chunk lane % 4, then permuted
  // (kq_perm8). Measured per format and GEMM: Q4_K gate-up 72 -> 62 us,
  // Q5_K 83 -> 73 us, Q8_0 135 -> 117 us; Q6_K (whose 2-aligned blocks take
  // 12-byte loads) and the down GEMMs (one wave per workgroup) measured
  // slower with them and load in MFMA order.
  constexpr bool CO = EPI == KQ_GATEUP && FMT != KQ_Q6_K;
  const int r16c = lane >> 2, kcc = lane & 3;
  const int psrc = (4 * r16 + kc) * 4;
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
  const int arow = act_row(r16), arow_c = act_row(r16c);
  int crow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) crow[i] = act_row(kc * 4 + i);

  const size_t a_rows = (size_t)g.a_rows;
  const __amdgpu_buffer_rsrc_t rq = kq_rsrc(g.xq, a_rows * g.kdim);
  const __amdgpu_buffer_rsrc_t rd =
      kq_rsrc(g.xd, FMT == KQ_Q8_0 ? a_rows * (g.kdim / 32) * 2 : a_rows * nsb * 4);
  const __amdgpu_buffer_rsrc_t rs =
      kq_rsrc(g.xs, FMT == KQ_Q8_0 ? 0 : a_rows * (g.kdim / 16) * 4);
  const size_t row_bytes = (size_t)nsb * UB;
  const __amdgpu_buffer_rsrc_t rw =
      kq_rsrc(g.W + (size_t)e * g.b_rows * row_bytes, (size_t)g.b_rows * row_bytes);

  // byte offsets (unit 0) of this lane's weight rows: fragment f is column
  // group f / 2 (gate-up: f even gate, f odd up) or f (down)
  uint32_t wrow[NB], wrow_c[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f) {
    const int fo = (EPI == KQ_GATEUP) ? (f >> 1) : f;
    const int c = col0 + fo * 16 + r16, cc = col0 + fo * 16 + r16c;
    const int wr = (EPI == KQ_GATEUP && (f & 1)) ? g.n_out + c : c;
    const int wrc = (EPI == KQ_GATEUP && (f & 1)) ? g.n_out + cc : cc;
    wrow[f] = (c < g.n_out) ? (uint32_t)(wr * row_bytes) : kqOob;
    wrow_c[f] = (cc < g.n_out) ? (uint32_t)(wrc * row_bytes) : kqOob;
  }

  float acc[NB][4];
#pragma unroll
  for (int f = 0; f < NB; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[f][i] = 0.0f;

  // this wave's units
  const int per = (nsb + KS - 1) / KS;
  const int u0 = min(nsb, wave * per), u1 = min(nsb, u0 + per);
  for (int u = u0; u < u1; ++u) {
    KqA<FMT> a;
    kq_aload<FMT, CO>(a, g, rq, rd, rs, arow, crow, u, kc, arow_c, kcc, psrc);
    // Q6_K: activation operands restricted to k 0-15 / 16-31 of each group
    long alo[8], ahi[8];
    if constexpr (FMT == KQ_Q6_K) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        alo[j] = (kc < 2) ? a.aop[j] : 0;
        ahi[j] = (kc < 2) ? 0 : a.aop[j];
      }
    }
    KqW<FMT> w[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f)
      kq_wload<FMT, CO>(w[f], rw, wrow[f] + (uint32_t)u * UB, kc, wrow_c[f] + (uint32_t)u * UB,
                        kcc, psrc);
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      // one fragment at a time: keeps the MFMA results of only one
      // fragment live
      __builtin_amdgcn_sched_barrier(0);
      kq_frag<FMT>(acc[f], w[f], a, alo, ahi, kc);
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

hipError_t launch_quantize_q8_0(const uint16_t* x, int R, int K, int8_t* qs, uint16_t* d,
                                hipStream_t s) {
  const long long nblk = (long long)R * (K / 32);
  const long long threads = nblk * 4;
  hipLaunchKernelGGL(quantize_q8_0_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, x, nblk, qs, d);
  return hipGetLastError();
}

template <int EPI, int FMT, int KS, int NFO>
static hipError_t kq_launch_shape(KqArgs g, hipStream_t s) {
  g.nblk = (g.n_out + 16 * NFO - 1) / (16 * NFO);
  g.slots = kq_slots(g.P, g.E, g.offsets != nullptr);
  const unsigned grid = (unsigned)((long long)g.slots * g.nblk);
  void* args[] = {&g};
  return timed_launch(reinterpret_cast<const void*>(kq_stream_kernel<EPI, FMT, KS, NFO>),
                      dim3(grid), dim3(64 * KS), args, s);
}

// 32 output columns per workgroup. Gate-up (H units of 256, two weight rows
// per column) splits k over up to 4 waves; down (fewer units, twice the
// columns) gives each workgroup one wave and all the units, which measured
// faster on the decode shapes.
template <int EPI, int FMT>
static hipError_t kq_launch_fmt(KqArgs g, hipStream_t s) {
  if constexpr (EPI == KQ_DOWN) {
    return kq_launch_shape<EPI, FMT, 1, 2>(g, s);
  } else {
    const int nsb = g.kdim / kQK;
    if (nsb >= 4) return kq_launch_shape<EPI, FMT, 4, 2>(g, s);
    if (nsb == 3) return kq_launch_shape<EPI, FMT, 3, 2>(g, s);
    if (nsb == 2) return kq_launch_shape<EPI, FMT, 2, 2>(g, s);
    return kq_launch_shape<EPI, FMT, 1, 2>(g, s);
  }
}

template <int EPI>
static hipError_t kq_launch(KqArgs g, int wtype, hipStream_t s) {
  switch (wtype) {
    case KQ_Q4_K: return kq_launch_fmt<EPI, KQ_Q4_K>(g, s);
    case KQ_Q5_K: return kq_launch_fmt<EPI, KQ_Q5_K>(g, s);
    case KQ_Q6_K: return kq_launch_fmt<EPI, KQ_Q6_K>(g, s);
    case KQ_Q8_0: return kq_launch_fmt<EPI, KQ_Q8_0>(g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_kq_gateup_silu(const int8_t* xq, const void* xd, const int32_t* xs, int T, int H,
                                 const uint8_t* w_gu, int wtype, int E, int I,
                                 const int32_t* sorted, const int32_t* offsets, int K,
                                 uint16_t* act, hipStream_t s) {
  KqArgs g{};
  g.xq = xq; g.xd = xd; g.xs = xs; g.a_rows = T;
  g.sorted = sorted; g.gather_k = K;
  g.W = w_gu; g.b_rows = 2 * I;
  g.offsets = offsets; g.E = E; g.P = T * K; g.kdim = H; g.n_out = I;
  g.out = act;
  return kq_launch<KQ_GATEUP>(g, wtype, s);
}

hipError_t launch_kq_down(const int8_t* aq, const void* ad, const int32_t* as, int P, int I,
                          const uint8_t* w_d, int wtype, int E, int H, const int32_t* sorted,
                          const int32_t* offsets, const float* pair_w, uint16_t* out,
                          hipStream_t s) {
  KqArgs g{};
  g.xq = aq; g.xd = ad; g.xs = as; g.a_rows = P;
  g.sorted = sorted; g.gather_k = 0;
  g.W = w_d; g.b_rows = H;
  g.offsets = offsets; g.E = E; g.P = P; g.kdim = I; g.n_out = H;
  g.out = out; g.pair_w = pair_w;
  return kq_launch<KQ_DOWN>(g, wtype, s);
}

}  // namespace moe
