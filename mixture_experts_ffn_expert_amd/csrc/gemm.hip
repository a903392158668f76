// gemm.hip -- grouped BF16 expert GEMMs on gfx950 MFMA.
//
// The operations are the two BF16 grouped expert GEMMs of vllm.cpp issue
// #3094 (row "BACKEND-ROCM-BF16-MOE", row statement) with its numeric
// contract: the gate-up result is narrowed to bf16 before SiLU-mul (N1) and
// the routing weight multiplies the f32 down-projection accumulator before
// the one bf16 rounding of the store (N2), so the combine never applies it
// again (N3). Rows are grouped per expert (PR #523 What changed: the grouped
// op runs over the rows' expert ids).
//
// Every GEMM here is C[m, n] = sum_k A[m, k] * B[n, k]: both operands are
// k-contiguous rows (activations [rows, k], weights [E, n, k]), the friendly
// layout for MFMA, where every lane loads 8 consecutive bf16 of one row.
//
// Work decomposition. The rows of expert e are offsets[e] .. offsets[e+1]
// of the sorted order. A "tile slot" is one BM-row block of one expert;
// slots are numbered expert after expert, and every workgroup finds its
// expert by a wavefront scan of the per-expert tile counts (experts with no
// rows own no slot and cost nothing). The host sizes the grid from the bound
// ceil(P/BM) + min(E, P) on the number of slots; surplus workgroups leave at
// once.
//
// Two kernel shapes:
//  * stream_kernel (few rows per expert, e.g. decode): one wave owns a 16- or
//    32-row block and a slab of output columns over the whole k range. Each
//    weight element is used by exactly one wave, so weights go straight from
//    HBM into MFMA operand registers (v_mfma_f32_16x16x32_bf16) with no LDS
//    and no barrier in the k loop; the k loop is unrolled so each wave keeps
//    several KiB of loads in flight. HBM-bound by design.
//  * tiled_kernel (hundreds of rows per expert, prefill): 128 x 128 block
//    tile, 4 waves of 64 x 64, k step 64 staged through LDS with padded rows
//    (conflict-free 16-byte reads), register prefetch of the next k step
//    during the MFMAs (v_mfma_f32_32x32x16_bf16).
//
// Epilogues (all per element, f32, no contraction):
//  * gate-up: the block loads the gate rows [n, n+16) / [n, n+32) and the
//    matching up rows I+[n, ...) as paired MFMA fragments, so one lane holds
//    gate and up of the same (row, column): act = bf16(silu(bf16(g)) * bf16(u)).
//  * down: bf16(acc * pair_w[p]) stored at pair row p = sorted[q].
//  * f32: acc (+ bias) stored as f32 (router and gate logits).
#include "device_math.h"
#include "launch.h"

namespace moe {

enum { EPI_GATEUP = 0, EPI_DOWN = 1, EPI_F32 = 2 };

struct GemmArgs {
  const uint16_t* A;        // activation rows: x [a_rows, kdim] (gathered) or act [P, kdim]
  int a_rows;               // rows of A (bounds of the gather)
  const int32_t* sorted;    // sorted pair ids, or null (row q of the problem is row q of A)
  int gather_k;             // >0: A row = sorted[q] / gather_k (gate-up); 0: A row = q
  const uint16_t* B;        // weights [E, b_rows, kdim]
  int b_rows;               // rows per expert in B (2I gate-up, H down, N logits)
  const int32_t* offsets;   // [E+1] expert row offsets, or null (one expert, P rows)
  int E, P, kdim;
  int n_out;                // output columns (I gate-up, H down, N logits)
  void* out;                // act bf16 [P, I] / expert_out bf16 [P, H] / f32 [P, N]
  const float* pair_w;      // down: f32 [P] or null
  const float* bias;        // f32: [N] or null
  int slots;                // tile slots in the grid
  int nblk;                 // column blocks in the grid
};

// Finds tile slot `slot` (BM rows) of the grouped problem. Must be called by
// a whole wavefront; the result is uniform across it.
__device__ __forceinline__ bool find_tile(const GemmArgs& g, int BM, int slot, int& e, int& row0,
                                          int& rows) {
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
    const bool mine = nt > 0 && slot >= first && slot < first + nt;
    const uint64_t hit = __ballot(mine);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      e = __shfl(ex, src);
      const int f = __shfl(first, src);
      const int oo = __shfl(o0, src);
      const int cc = __shfl(cnt, src);
      row0 = oo + (slot - f) * BM;
      rows = min(BM, cc - (slot - f) * BM);
      return true;
    }
    before += __shfl(incl, 63);
  }
  return false;
}

// Pointer to the A row of problem row q (null: zero row).
__device__ __forceinline__ const uint16_t* a_row_ptr(const GemmArgs& g, int q) {
  int r = q;
  if (g.sorted != nullptr && g.gather_k > 0) {
    const int p = g.sorted[q];
    if (p < 0) return nullptr;
    r = p / g.gather_k;
  }
  if (r < 0 || r >= g.a_rows) return nullptr;
  return g.A + (size_t)r * g.kdim;
}

// B row of output column c for fragment kind (0: gate/plain, 1: up).
template <int EPI>
__device__ __forceinline__ const uint16_t* b_row_ptr(const GemmArgs& g, int e, int c, int up) {
  if (c >= g.n_out) return nullptr;
  const int r = (EPI == EPI_GATEUP && up) ? g.n_out + c : c;
  return g.B + ((size_t)e * g.b_rows + r) * g.kdim;
}

__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

__device__ __forceinline__ bf16x8_t zero8() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8_t, z);
}

// Epilogue of one output element (row q of the problem, column c).
template <int EPI>
__device__ __forceinline__ void store_plain(const GemmArgs& g, int q, int c, float acc) {
#pragma clang fp contract(off)
  if (EPI == EPI_DOWN) {
    const int p = (g.sorted != nullptr) ? g.sorted[q] : q;
    if (p < 0 || p >= g.P) return;
    float y = acc;
    if (g.pair_w != nullptr) y = y * g.pair_w[p];
    reinterpret_cast<uint16_t*>(g.out)[(size_t)p * g.n_out + c] = (uint16_t)f32_to_bf16(y);
  } else {
    float y = acc;
    if (g.bias != nullptr) y = y + g.bias[c];
    reinterpret_cast<float*>(g.out)[(size_t)q * g.n_out + c] = y;
  }
}

__device__ __forceinline__ void store_gateup(const GemmArgs& g, int q, int c, float gate,
                                             float up) {
#pragma clang fp contract(off)
  const float gb = round_bf16(gate);  // N1: narrow before the activation
  const float ub = round_bf16(up);
  const float v = silu_cw(gb) * ub;
  reinterpret_cast<uint16_t*>(g.out)[(size_t)q * g.n_out + c] = (uint16_t)f32_to_bf16(v);
}

// ---------------------------------------------------------------------------
// stream_kernel: MF 16-row fragments x NFO 16-column output fragments per wave
// ---------------------------------------------------------------------------
template <int EPI, int MF, int NFO>
__global__ __launch_bounds__(256) void stream_kernel(GemmArgs g) {
  constexpr int NB = (EPI == EPI_GATEUP) ? 2 * NFO : NFO;  // B fragments per wave
  constexpr int BM = 16 * MF;
  constexpr int COLS_PER_WAVE = 16 * NFO;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int blk = blockIdx.x;
  const int slot = blk / g.nblk;
  const int nb = blk - slot * g.nblk;
  int e, row0, rows;
  if (!find_tile(g, BM, slot, e, row0, rows)) return;
  const int col0 = (nb * 4 + wave) * COLS_PER_WAVE;
  if (col0 >= g.n_out) return;

  const int r16 = lane & 15;
  const int kc = (lane >> 4) * 8;
  const uint16_t* pa[MF];
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int rr = i * 16 + r16;
    pa[i] = (rr < rows) ? a_row_ptr(g, row0 + rr) : nullptr;
  }
  const uint16_t* pb[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f) {
    const int fo = (EPI == EPI_GATEUP) ? (f >> 1) : f;
    const int up = (EPI == EPI_GATEUP) ? (f & 1) : 0;
    pb[f] = b_row_ptr<EPI>(g, e, col0 + fo * 16 + r16, up);
  }
  f32x4_t acc[MF][NB];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int U = 4;  // k steps of 32 per unrolled iteration
  const int kmain = (g.kdim / (32 * U)) * (32 * U);
  int k0 = 0;
  for (; k0 < kmain; k0 += 32 * U) {
    bf16x8_t a[U][MF], b[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int f = 0; f < NB; ++f)
        b[u][f] = pb[f] ? load8(pb[f] + k0 + u * 32 + kc) : zero8();
#pragma unroll
      for (int i = 0; i < MF; ++i)
        a[u][i] = pa[i] ? load8(pa[i] + k0 + u * 32 + kc) : zero8();
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int f = 0; f < NB; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][i], b[u][f], acc[i][f], 0, 0, 0);
  }
  for (; k0 < g.kdim; k0 += 32) {  // tail: 8-element chunks past kdim read as zero
    const bool in = k0 + kc < g.kdim;
    bf16x8_t a[MF], b[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) b[f] = (in && pb[f]) ? load8(pb[f] + k0 + kc) : zero8();
#pragma unroll
    for (int i = 0; i < MF; ++i) a[i] = (in && pa[i]) ? load8(pa[i] + k0 + kc) : zero8();
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int f = 0; f < NB; ++f)
        acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[f], acc[i][f], 0, 0, 0);
  }

  // C layout of 16x16: element r of lane l is row (l/16)*4 + r, column l%16
#pragma unroll
  for (int i = 0; i < MF; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = i * 16 + (lane >> 4) * 4 + r;
      if (rr >= rows) continue;
      const int q = row0 + rr;
#pragma unroll
      for (int fo = 0; fo < NFO; ++fo) {
        const int c = col0 + fo * 16 + r16;
        if (c >= g.n_out) continue;
        if (EPI == EPI_GATEUP)
          store_gateup(g, q, c, acc[i][2 * fo][r], acc[i][2 * fo + 1][r]);
        else
          store_plain<EPI>(g, q, c, acc[i][fo][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// tiled_kernel: 128 x 128 tile, 4 waves (2 x 2) of 64 x 64, k step 64 in LDS
// ---------------------------------------------------------------------------
constexpr int TBM = 128, TBN = 128, TBK = 64, TLD = TBK + 8;

template <int EPI>
__global__ __launch_bounds__(256) void tiled_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t As[TBM * TLD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[TBN * TLD];
  __shared__ int tile_info[3];
  constexpr int OUT_COLS = (EPI == EPI_GATEUP) ? TBN / 2 : TBN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int blk = blockIdx.x;
  const int slot = blk / g.nblk;
  const int nb = blk - slot * g.nblk;
  if (wave == 0) {
    int e = 0, row0 = 0, rows = 0;
    if (!find_tile(g, TBM, slot, e, row0, rows)) rows = 0;
    if (lane == 0) {
      tile_info[0] = e;
      tile_info[1] = row0;
      tile_info[2] = rows;
    }
  }
  __syncthreads();
  const int e = tile_info[0], row0 = tile_info[1], rows = tile_info[2];
  if (rows <= 0) return;
  const int n0 = nb * OUT_COLS;

  // global -> LDS assignment: 8 threads per 64-element row, 32 rows per pass
  const int lc = (tid & 7) * 8;
  const uint16_t* ga[4];
  const uint16_t* gb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    ga[i] = (r < rows) ? a_row_ptr(g, row0 + r) : nullptr;
    int c, up = 0;
    if (EPI == EPI_GATEUP) {
      const int wn = r >> 6, f = (r >> 5) & 1, j = r & 31;
      c = n0 + wn * 32 + j;
      up = f;
    } else {
      c = n0 + r;
    }
    gb[i] = b_row_ptr<EPI>(g, e, c, up);
  }

  const int wm = wave & 1, wn = wave >> 1;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  bf16x8_t ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = k0 + lc < g.kdim;
      ra[i] = (in && ga[i]) ? load8(ga[i] + k0 + lc) : zero8();
      rb[i] = (in && gb[i]) ? load8(gb[i] + k0 + lc) : zero8();
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<bf16x8_t*>(&As[r * TLD + lc]) = ra[i];
      *reinterpret_cast<bf16x8_t*>(&Bs[r * TLD + lc]) = rb[i];
    }
  };

  const int nk = (g.kdim + TBK - 1) / TBK;
  gload(0);
  const int r32 = lane & 31;
  const int kh = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (kt + 1 < nk) gload((kt + 1) * TBK);
#pragma unroll
    for (int kk = 0; kk < TBK / 16; ++kk) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 64 + i * 32 + r32) * TLD + kk * 16 + kh]);
#pragma unroll
      for (int f = 0; f < 2; ++f)
        b[f] = *reinterpret_cast<const bf16x8_t*>(&Bs[(wn * 64 + f * 32 + r32) * TLD + kk * 16 + kh]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int f = 0; f < 2; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[f], acc[i][f], 0, 0, 0);
    }
  }

  // C layout of 32x32: element r of lane l is row (r/4)*8 + (l/32)*4 + r%4, column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (rr >= rows) continue;
      const int q = row0 + rr;
      if (EPI == EPI_GATEUP) {
        const int c = n0 + wn * 32 + r32;
        if (c < g.n_out) store_gateup(g, q, c, acc[i][0][r], acc[i][1][r]);
      } else {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int c = n0 + wn * 64 + f * 32 + r32;
          if (c < g.n_out) store_plain<EPI>(g, q, c, acc[i][f][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
static inline int slots_for(int P, int E, int BM, bool grouped) {
  const int full = (P + BM - 1) / BM;
  return grouped ? full + (E < P ? E : P) : full;
}

template <int EPI>
static hipError_t dispatch(GemmArgs g, hipStream_t s) {
  const bool grouped = g.offsets != nullptr;
  const double avg_rows = grouped ? (double)g.P / (double)g.E : (double)g.P;
  if (avg_rows <= 24.0) {
    // few rows per expert: weight streaming, one wave per 16 (or 32) rows x 32 columns
    constexpr int NFO = (EPI == EPI_GATEUP) ? 1 : 2;
    const int cols_per_block = 4 * 16 * NFO;
    g.nblk = (g.n_out + cols_per_block - 1) / cols_per_block;
    if (avg_rows <= 8.0) {
      g.slots = slots_for(g.P, g.E, 16, grouped);
      hipLaunchKernelGGL((stream_kernel<EPI, 1, NFO>), dim3(g.slots * g.nblk), dim3(256), 0, s, g);
    } else {
      g.slots = slots_for(g.P, g.E, 32, grouped);
      hipLaunchKernelGGL((stream_kernel<EPI, 2, NFO>), dim3(g.slots * g.nblk), dim3(256), 0, s, g);
    }
  } else {
    const int out_cols = (EPI == EPI_GATEUP) ? TBN / 2 : TBN;
    g.nblk = (g.n_out + out_cols - 1) / out_cols;
    g.slots = slots_for(g.P, g.E, TBM, grouped);
    hipLaunchKernelGGL((tiled_kernel<EPI>), dim3(g.slots * g.nblk), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_gateup_silu(const uint16_t* x, int T, int H, const uint16_t* w_gu, int E, int I,
                              const int32_t* sorted, const int32_t* offsets, int K, uint16_t* act,
                              hipStream_t s) {
  GemmArgs g{};
  g.A = x;
  g.a_rows = T;
  g.sorted = sorted;
  g.gather_k = K;
  g.B = w_gu;
  g.b_rows = 2 * I;
  g.offsets = offsets;
  g.E = E;
  g.P = T * K;
  g.kdim = H;
  g.n_out = I;
  g.out = act;
  return dispatch<EPI_GATEUP>(g, s);
}

hipError_t launch_down(const uint16_t* act, int P, int I, const uint16_t* w_d, int E, int H,
                       const int32_t* sorted, const int32_t* offsets, const float* pair_w,
                       uint16_t* expert_out, hipStream_t s) {
  GemmArgs g{};
  g.A = act;
  g.a_rows = P;
  g.sorted = sorted;
  g.gather_k = 0;  // act is already in sorted order: row q of the problem is row q of act
  g.B = w_d;
  g.b_rows = H;
  g.offsets = offsets;
  g.E = E;
  g.P = P;
  g.kdim = I;
  g.n_out = H;
  g.out = expert_out;
  g.pair_w = pair_w;
  return dispatch<EPI_DOWN>(g, s);
}

hipError_t launch_logits(const uint16_t* x, int T, int H, const uint16_t* w, int N,
                         const float* bias, float* out, hipStream_t s) {
  GemmArgs g{};
  g.A = x;
  g.a_rows = T;
  g.sorted = nullptr;
  g.gather_k = 0;
  g.B = w;
  g.b_rows = N;
  g.offsets = nullptr;
  g.E = 1;
  g.P = T;
  g.kdim = H;
  g.n_out = N;
  g.out = out;
  g.bias = bias;
  return dispatch<EPI_F32>(g, s);
}

}  // namespace moe
