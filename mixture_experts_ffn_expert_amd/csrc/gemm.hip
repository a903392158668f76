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
// Every GEMM here is C[m, n] = sum_k A[m, k] * B[n, k]: activations are
// k-contiguous rows [rows, k]; expert weights W [E, n, k] arrive packed into
// 1 KiB blocks of 16 rows x 32 k in MFMA lane order (layout below, written
// once by pack.hip), so every weight load of a wavefront is one contiguous
// 1 KiB; the router weights stay plain rows.
//
// Work decomposition. The rows of expert e are offsets[e] .. offsets[e+1]
// of the sorted order. A "tile slot" is one BM-row block of one expert;
// slots are numbered expert after expert, and every workgroup finds its
// expert by a wavefront scan of the per-expert tile counts (experts with no
// rows own no slot and cost nothing). The host sizes the grid from the bound
// ceil(P/BM) + min(E, P) on the number of slots; surplus workgroups leave at
// once.
//
// Three kernels, picked on the host by rows per expert and tile count:
//  * stream_kernel (few rows per expert: decode, many small experts, a dense
//    shared expert of a few hundred rows): a workgroup owns a 16- or 32-row
//    block of one expert and 16..64 output columns; its waves split the k
//    range. Each weight element is used by exactly one wave, so weights go
//    straight from HBM into MFMA operand registers (v_mfma_f32_16x16x32_bf16)
//    with no LDS staging and no barrier in the k loop; the partial tiles meet
//    once in LDS, added in a fixed order. The small work units keep every CU
//    streaming to the end. HBM-bound by design.
//  * tiled_dma_kernel (gate-up and down with hundreds of rows per expert):
//    320 x 256 block tile on 8 waves (128 x 128 for a gate-up with too few
//    320-row tiles to fill the chip), k step 64, a 2-stage LDS ring filled by
//    direct-to-LDS buffer loads that four producer waves issue,
//    XOR-swizzled rows, v_mfma_f32_32x32x16_bf16, blocks regrouped by XCD;
//    the 32-row fragments past a tile's last row are skipped; the gate-up's
//    SiLU comes from a table that the stage past the end of k loads.
//  * tiled_kernel (a down GEMM with too few 320 x 256 tiles: an owner's
//    share): 128 x 128 block tile, 4 waves of 64 x 64, k step 64 staged
//    through LDS with padded rows (conflict-free 16-byte reads), register
//    prefetch of the next k step during the MFMAs, 4 workgroups per CU.
//
// Epilogues (all per element, f32, no contraction):
//  * gate-up: the block loads the gate rows [n, n+16) / [n, n+32) and the
//    matching up rows I+[n, ...) as paired MFMA fragments, so one lane holds
//    gate and up of the same (row, column): act = bf16(silu(bf16(g)) * bf16(u)).
//  * down: bf16(acc * pair_w[p]) stored at pair row p = sorted[q].
//  * f32: acc (+ bias) stored as f32 (router and gate logits).
#include <hip/hip_ext.h>

#include "device_math.h"
#include "launch.h"
#include "lds_dma.h"
#include "silu_table.h"

namespace moe {

// silu_cw of the 7,936 bf16 gate values without a closed form (silu_table.h),
// built by the compiler; 32 KiB of read-only device memory.
__constant__ SiluTable kSiluTable = make_silu_table();

enum { EPI_GATEUP = 0, EPI_DOWN = 1, EPI_F32 = 2 };

struct GemmArgs {
  const uint16_t* A;        // activation rows: x [a_rows, kdim] (gathered) or act [P, kdim]
  int a_rows;               // rows of A (bounds of the gather)
  const int32_t* sorted;    // sorted pair ids, or null (row q of the problem is row q of A)
  int gather_k;             // >0: A row = sorted[q] / gather_k (gate-up); 0: A row = q
  const uint16_t* B;        // weights: packed blocks (gate-up, down) or [N, kdim] (logits)
  uint32_t b_bytes;         // bytes of one expert's weights (packed or plain)
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

// Expert-major block order for the tiled kernel. Logical block L is mapped
// to (expert e, row tile mt of e, column block nb): experts in order; inside
// an expert, groups of GM row tiles (outer), column blocks (middle), row
// tiles of the group (inner). Consecutive blocks then reuse one weight tile
// across GM row tiles and one activation tile across the column blocks.
// Called by a whole wavefront; the result is uniform across it.
__device__ __forceinline__ bool find_block(const GemmArgs& g, int BM, int GM, int L, int& e,
                                           int& row0, int& rows, int& nb) {
  if (g.offsets == nullptr) {  // one expert, P rows
    const int mt_e = (g.P + BM - 1) / BM;
    if (L >= mt_e * g.nblk) return false;
    e = 0;
    const int full = mt_e / GM;
    int mg = L / (GM * g.nblk), gm = GM, rem = L - mg * GM * g.nblk;
    if (mg >= full) {
      mg = full;
      gm = mt_e - full * GM;
      rem = L - full * GM * g.nblk;
    }
    nb = rem / gm;
    const int mt = mg * GM + (rem - nb * gm);
    row0 = mt * BM;
    rows = min(BM, g.P - row0);
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
    const int mt_e = (cnt + BM - 1) / BM;
    const int nbl = mt_e * g.nblk;
    int incl = nbl;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(incl, m);
      if (lane >= m) incl += o;
    }
    const int first = before + incl - nbl;
    const bool mine = nbl > 0 && L >= first && L < first + nbl;
    const uint64_t hit = __ballot(mine);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      e = __builtin_amdgcn_readlane(ex, src);
      const int f = __builtin_amdgcn_readlane(first, src);
      const int oo = __builtin_amdgcn_readlane(o0, src);
      const int cc = __builtin_amdgcn_readlane(cnt, src);
      const int mte = __builtin_amdgcn_readlane(mt_e, src);
      const int local = L - f;
      const int full = mte / GM;
      int mg = local / (GM * g.nblk), gm = GM, rem = local - mg * GM * g.nblk;
      if (mg >= full) {
        mg = full;
        gm = mte - full * GM;
        rem = local - full * GM * g.nblk;
      }
      nb = rem / gm;
      const int mt = mg * GM + (rem - nb * gm);
      row0 = oo + mt * BM;
      rows = min(BM, cc - mt * BM);
      return true;
    }
    before += __builtin_amdgcn_readlane(incl, 63);
  }
  return false;
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

// COH: store as an agent-scope (relaxed) atomic, written through to the
// device's point of coherence (the fused FFN's act, read by other CUs).
template <bool COH = false>
__device__ __forceinline__ void store_gateup(const GemmArgs& g, int q, int c, float gate,
                                             float up) {
#pragma clang fp contract(off)
  const float gb = round_bf16(gate);  // N1: narrow before the activation
  const float ub = round_bf16(up);
  const float v = silu_cw(gb) * ub;
  uint16_t* p = reinterpret_cast<uint16_t*>(g.out) + (size_t)q * g.n_out + c;
  const uint16_t b = (uint16_t)f32_to_bf16(v);
  if constexpr (COH)
    __hip_atomic_store(p, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = b;
}

// ---------------------------------------------------------------------------
// Buffer loads. A raw buffer load whose byte offset lies past the resource's
// size returns zero without touching memory, so rows past the end of a tile,
// columns past n_out and k past kdim are read as zeros with no branch: every
// lane keeps one fixed byte offset (kOob for a zero row) and the k position
// goes into the scalar offset. Buffer sizes stay below 2^31 bytes (checked
// at the C ABI), so kOob plus any k offset stays out of range.
// ---------------------------------------------------------------------------
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ bf16x8_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// NT: the same load with the non-temporal hint (cache policy nt), for data
// read once per launch: the weights of a grouped expert whose rows fit one
// row tile of a streaming kernel. Decode gate-up 114.5 -> 103.0 us, down
// 58.8 -> 53.1 us. Weights that several row tiles read (a dense expert's, a
// busy expert's, the router's, and the tile kernels', whose workgroups share
// weight tiles through the caches) measured slower with it: cached loads.
template <bool NT>
__device__ __forceinline__ bf16x8_t wload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? 2 : 0));
}

// ---------------------------------------------------------------------------
// Packed expert weights (written once by moe_pack_weights, pack.hip). One
// expert's matrix W [R, kdim] is cut into 1 KiB blocks of 16 rows x 32 k;
// inside a block, 16-byte chunk q = 16 c + r holds W[16 rb + r][32 kb + 8 c ..
// + 8], the order in which the 64 lanes of a wavefront hold one 16 x 32 MFMA
// operand, so a block is one coalesced 64-lane load. Rows past R and k past
// kdim are zero. Down (and any plain) matrix: block (rb, kb) at
// (rb * nkb + kb) KiB. Gate-up [2I, kdim]: the gate block of output columns
// [16 cb, +16) and the matching up block (rows I + [16 cb, +16)) sit side by
// side: (cb, kb, f) at ((cb * nkb + kb) * 2 + f) KiB, f = 0 gate, 1 up.
// ---------------------------------------------------------------------------
// Byte offset of the A row of problem row q inside A (kOob: zero row).
__device__ __forceinline__ uint32_t a_row_off(const GemmArgs& g, int q) {
  int r = q;
  if (g.sorted != nullptr && g.gather_k > 0) {
    const int p = g.sorted[q];
    if (p < 0) return kOob;
    r = p / g.gather_k;
  }
  if (r < 0 || r >= g.a_rows) return kOob;
  return (uint32_t)r * (uint32_t)g.kdim * 2u;
}

// Byte offset of row c of a plain (row-major) weight matrix (logits).
__device__ __forceinline__ uint32_t b_row_off(const GemmArgs& g, int c) {
  if (c >= g.n_out) return kOob;
  return (uint32_t)c * (uint32_t)g.kdim * 2u;
}

// Packed expert weights. Byte offset, at k block 0, of the 1 KiB block
// holding output columns [16 cb, 16 cb + 16) (gate-up: gate half f = 0 or
// up half f = 1); consecutive k blocks follow kb_stride<EPI>() bytes apart.
template <int EPI>
__device__ __forceinline__ uint32_t b_block_off(const GemmArgs& g, int cb, int f) {
  if (cb * 16 >= g.n_out) return kOob;
  const uint32_t nkb = (uint32_t)packed_nkb(g.kdim);
  if (EPI == EPI_GATEUP) return ((uint32_t)cb * nkb * 2u + (uint32_t)f) * kPackBlock;
  return (uint32_t)cb * nkb * kPackBlock;
}
template <int EPI>
__device__ __forceinline__ constexpr uint32_t kb_stride() {
  return EPI == EPI_GATEUP ? 2u * kPackBlock : kPackBlock;
}

// ---------------------------------------------------------------------------
// stream_kernel: one workgroup = 16*MF rows x 16*NFO output columns; its KS
// waves split the k range into contiguous parts and add their partial tiles
// in LDS in a fixed wave order (deterministic). Splitting k makes the work
// units small enough to balance HBM streaming across all CUs.
// ---------------------------------------------------------------------------
// The body, for workgroup `blk` of the grid: false when its slot holds no
// tile (uniform over the workgroup; nothing done then).
template <int EPI, int MF, int NFO, int KS>
constexpr int stream_red_floats() {
  return KS * MF * ((EPI == EPI_GATEUP) ? 2 * NFO : NFO) * 4 * 64;
}

// The k loop of one wave of stream_body over [kb, ke): U 32-wide k steps of
// loads in flight, then their MFMAs; the weight loads non-temporal if NTL.
template <bool NTL, int MF, int NB, int U, typename BSoff>
__device__ __forceinline__ void stream_kloop(f32x4_t (&acc)[MF][NB], __amdgpu_buffer_rsrc_t ra_rsrc,
                                             __amdgpu_buffer_rsrc_t rb_rsrc,
                                             const uint32_t (&va)[MF], const uint32_t (&vb)[NB],
                                             BSoff bsoff, int kb, int ke, int kc) {
  int k0 = kb;
  for (; k0 + 32 * U <= ke; k0 += 32 * U) {
    bf16x8_t a[U][MF], b[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t soff = (uint32_t)(k0 + u * 32) * 2u;
      const uint32_t sb = bsoff(k0 + u * 32);
#pragma unroll
      for (int f = 0; f < NB; ++f) b[u][f] = wload8<NTL>(rb_rsrc, vb[f], sb);
#pragma unroll
      for (int i = 0; i < MF; ++i) a[u][i] = bload8(ra_rsrc, va[i], soff);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int f = 0; f < NB; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][i], b[u][f], acc[i][f], 0, 0, 0);
  }
  for (; k0 < ke; k0 += 32) {  // tail: 8-element chunks at or past ke read as zero
    const bool in = k0 + kc < ke;
    const uint32_t soff = (uint32_t)k0 * 2u;
    bf16x8_t a[MF], b[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) b[f] = wload8<NTL>(rb_rsrc, in ? vb[f] : kOob, bsoff(k0));
#pragma unroll
    for (int i = 0; i < MF; ++i) a[i] = bload8(ra_rsrc, in ? va[i] : kOob, soff);
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int f = 0; f < NB; ++f)
        acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[f], acc[i][f], 0, 0, 0);
  }
}

// red: LDS of stream_red_floats<EPI, MF, NFO, KS>() floats for the partial
// tiles of the k waves.
template <int EPI, int MF, int NFO, int KS, int U, bool COH = false, bool NT = false>
__device__ __forceinline__ bool stream_body(const GemmArgs& g, int blk, float* red) {
  constexpr int NB = (EPI == EPI_GATEUP) ? 2 * NFO : NFO;  // B fragments per wave
  constexpr int BM = 16 * MF;
  auto R = [&](int w, int i, int f, int r) -> float& {
    return red[(((w * MF + i) * NB + f) * 4 + r) * 64 + (threadIdx.x & 63)];
  };
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = blk / g.nblk;
  const int nb = blk - slot * g.nblk;
  int e, row0, rows;
  if (!find_tile(g, BM, slot, e, row0, rows)) return false;  // uniform over the workgroup
  const int col0 = nb * 16 * NFO;

  // MFMA lane order of an operand: lane l holds row l % 16, k chunk l / 16
  const int r16 = lane & 15;
  const int kc = (lane >> 4) * 8;
  // Plain-row operands (both sides of the logits) are loaded coalesced
  // instead: four consecutive lanes read one row's 64 bytes (row l / 4,
  // chunk l % 4), and a lane permutation puts them in MFMA order. Loaded in
  // MFMA order, the 64 lanes of a load touch 64 separate 16-byte pieces.
  constexpr bool PACKED = EPI != EPI_F32;
  const int lr16 = PACKED ? r16 : (lane >> 2);
  const int lkc = PACKED ? kc : (lane & 3) * 8;
  const int perm_src = (4 * (lane & 15) + (lane >> 4)) * 4;  // ds_bpermute byte index
  auto to_mfma = [&](bf16x8_t v) -> bf16x8_t {
    if constexpr (PACKED) return v;
    u32x4_t u = __builtin_bit_cast(u32x4_t, v);
    u.x = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_src, (int)u.x);
    u.y = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_src, (int)u.y);
    u.z = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_src, (int)u.z);
    u.w = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_src, (int)u.w);
    return __builtin_bit_cast(bf16x8_t, u);
  };
  const __amdgpu_buffer_rsrc_t ra_rsrc =
      make_rsrc(g.A, (uint32_t)g.a_rows * (uint32_t)g.kdim * 2u);
  const __amdgpu_buffer_rsrc_t rb_rsrc =
      make_rsrc(reinterpret_cast<const unsigned char*>(g.B) + (size_t)e * g.b_bytes, g.b_bytes);
  uint32_t va[MF];
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int rr = i * 16 + lr16;
    va[i] = ((rr < rows) ? a_row_off(g, row0 + rr) : kOob) + lkc * 2;
  }
  // B: plain rows for the logits (k position in the scalar offset); packed
  // blocks for the expert weights, where lane l's 16 bytes of a 32-wide k
  // step are the l-th chunk of one 1 KiB block
  uint32_t vb[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f) {
    const int fo = (EPI == EPI_GATEUP) ? (f >> 1) : f;
    if constexpr (PACKED) {
      const uint32_t o = b_block_off<EPI>(g, col0 / 16 + fo, f & 1);
      vb[f] = (o == kOob) ? kOob : o + lane * 16;
    } else {
      vb[f] = b_row_off(g, col0 + fo * 16 + lr16) + lkc * 2;
    }
  }
  // scalar B offset of the 32-wide k step starting at k
  auto bsoff = [&](int k) -> uint32_t {
    if constexpr (PACKED) return (uint32_t)(k >> 5) * kb_stride<EPI>();
    return (uint32_t)k * 2u;
  };
  f32x4_t acc[MF][NB];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // this wave's k range: a multiple of 32 elements (the last one may be short)
  const int ksteps = (g.kdim + 31) >> 5;
  const int kper = ((ksteps + KS - 1) / KS) * 32;
  const int kb = min(g.kdim, __builtin_amdgcn_readfirstlane(wave) * kper);
  const int ke = min(g.kdim, kb + kper);
  // NT: the weight loads of a tile that is its expert's only one go out
  // non-temporal (no other workgroup reads those weights); an expert with
  // several row tiles has its weights re-read by each, through the caches.
  if constexpr (NT) {
    // the tile is its expert's only one when it starts at the expert's first
    // row and ends at its last (uniform over the workgroup); a dense expert
    // (no offsets: identity rows) is read by every row tile
    bool once = false;
    if (g.offsets != nullptr) {
      const int o0 = __builtin_amdgcn_readfirstlane(g.offsets[e]);
      const int o1 = __builtin_amdgcn_readfirstlane(g.offsets[e + 1]);
      once = row0 == o0 && row0 + rows == o1;
    }
    if (once)
      stream_kloop<true, MF, NB, U>(acc, ra_rsrc, rb_rsrc, va, vb, bsoff, kb, ke, kc);
    else
      stream_kloop<false, MF, NB, U>(acc, ra_rsrc, rb_rsrc, va, vb, bsoff, kb, ke, kc);
  } else {
    // (written out here rather than through stream_kloop: the router-logit
    // shapes keep 16 fewer VGPRs this way)
    int k0 = kb;
    for (; k0 + 32 * U <= ke; k0 += 32 * U) {
      bf16x8_t a[U][MF], b[U][NB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t soff = (uint32_t)(k0 + u * 32) * 2u;
        const uint32_t sb = bsoff(k0 + u * 32);
#pragma unroll
        for (int f = 0; f < NB; ++f) b[u][f] = bload8(rb_rsrc, vb[f], sb);
#pragma unroll
        for (int i = 0; i < MF; ++i) a[u][i] = bload8(ra_rsrc, va[i], soff);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int f = 0; f < NB; ++f) b[u][f] = to_mfma(b[u][f]);
#pragma unroll
        for (int i = 0; i < MF; ++i) a[u][i] = to_mfma(a[u][i]);
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int f = 0; f < NB; ++f)
            acc[i][f] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][i], b[u][f], acc[i][f], 0, 0, 0);
      }
    }
    for (; k0 < ke; k0 += 32) {  // tail: 8-element chunks at or past ke read as zero
      const bool in = k0 + lkc < ke;
      const uint32_t soff = (uint32_t)k0 * 2u;
      bf16x8_t a[MF], b[NB];
#pragma unroll
      for (int f = 0; f < NB; ++f) b[f] = to_mfma(bload8(rb_rsrc, in ? vb[f] : kOob, bsoff(k0)));
#pragma unroll
      for (int i = 0; i < MF; ++i) a[i] = to_mfma(bload8(ra_rsrc, in ? va[i] : kOob, soff));
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int f = 0; f < NB; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[f], acc[i][f], 0, 0, 0);
    }
  }

#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int f = 0; f < NB; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) R(wave, i, f, r) = acc[i][f][r];
  __syncthreads();

  // C layout of 16x16: element r of lane l is row (l/16)*4 + r, column l%16.
  // Wave w finishes the elements r = w, w + KS, ...: sum over waves 0..KS-1.
  for (int r = wave; r < 4; r += KS) {
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int rr = i * 16 + (lane >> 4) * 4 + r;
      float sum[NB];
#pragma unroll
      for (int f = 0; f < NB; ++f) {
        float s = R(0, i, f, r);
#pragma unroll
        for (int w = 1; w < KS; ++w) s = s + R(w, i, f, r);  // fixed order
        sum[f] = s;
      }
      if (rr >= rows) continue;
      const int q = row0 + rr;
#pragma unroll
      for (int fo = 0; fo < NFO; ++fo) {
        const int c = col0 + fo * 16 + r16;
        if (c >= g.n_out) continue;
        if (EPI == EPI_GATEUP)
          store_gateup<COH>(g, q, c, sum[2 * fo], sum[2 * fo + 1]);
        else
          store_plain<EPI>(g, q, c, sum[fo]);
      }
    }
  }
  return true;
}

template <int EPI, int MF, int NFO, int KS, int U, bool NT = false>
__global__ __launch_bounds__(64 * KS) void stream_kernel(GemmArgs g) {
  __shared__ float red[stream_red_floats<EPI, MF, NFO, KS>()];
  stream_body<EPI, MF, NFO, KS, U, false, NT>(g, blockIdx.x, red);
}

// ---------------------------------------------------------------------------
// tiled_kernel: BM x BN block tile (BN weight rows), WM x WN waves, k step BK
// staged through LDS with padded rows (BK = 64: 144-byte rows, conflict-free
// 16-byte fragment reads). The next k step is loaded into registers while
// the current one is multiplied (v_mfma_f32_32x32x16_bf16).
// ---------------------------------------------------------------------------
template <int EPI, int BM, int BN, int BK, int WM, int WN, int PF = 1, int MINB = 1, int GM = 0>
__global__ __launch_bounds__(64 * WM * WN, MINB) void tiled_kernel(GemmArgs g) {
  constexpr int NT = 64 * WM * WN;             // threads
  constexpr int TM = BM / WM, TN = BN / WN;    // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;    // 32x32 fragments per wave
  constexpr int LD = BK + 8;                   // padded LDS row (elements)
  constexpr int CPR = BK / 8;                  // 16-byte chunks per row
  constexpr int A_CH = BM * CPR / NT;          // chunks per thread
  constexpr int B_CH = BN * CPR / NT;
  constexpr int OUT_COLS = (EPI == EPI_GATEUP) ? BN / 2 : BN;
  static_assert(A_CH * NT == BM * CPR && B_CH * NT == BN * CPR, "tile / thread mismatch");
  static_assert(EPI != EPI_GATEUP || FN % 2 == 0, "gate-up pairs fragments");
  static_assert(EPI != EPI_F32, "logits use the streaming kernel");
  // Output staging: the bf16 result tile goes through LDS (reusing the
  // operand buffers) in NP passes of BM/NP rows, then leaves as 16-byte row
  // segments.
  constexpr int CLD = OUT_COLS + 8;                              // padded row (elements)
  constexpr int NP = (BM * CLD > (BM + BN) * LD) ? 2 : 1;
  static_assert(BM % (NP * 32 * 1) == 0 && (BM / NP) * CLD <= (BM + BN) * LD, "staging");
  __shared__ __attribute__((aligned(16))) uint16_t smem[(BM + BN) * LD];
  uint16_t* As = smem;
  uint16_t* Bs = smem + BM * LD;
  __shared__ int row_dest[BM];      // output row of each tile row (-1: none)
  __shared__ float row_w[BM];       // routing weight of each tile row (down)
  __shared__ int tile_info[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = blockIdx.x;
  if (wave == 0) {
    int e = 0, row0 = 0, rows = 0, nb = 0;
    bool ok;
    if (GM > 0) {
      ok = find_block(g, BM, GM, L, e, row0, rows, nb);
    } else {
      const int slot = L / g.nblk;
      nb = L - slot * g.nblk;
      ok = find_tile(g, BM, slot, e, row0, rows);
    }
    if (!ok) rows = 0;
    if (lane == 0) {
      tile_info[0] = e;
      tile_info[1] = row0;
      tile_info[2] = rows;
      tile_info[3] = nb;
    }
  }
  __syncthreads();
  const int e = tile_info[0], row0 = tile_info[1], rows = tile_info[2], nb = tile_info[3];
  if (rows <= 0) return;
  const int n0 = nb * OUT_COLS;
  for (int rr = tid; rr < BM; rr += NT) {
    int dest = -1;
    float wgt = 1.0f;
    if (rr < rows) {
      const int q = row0 + rr;
      dest = q;
      if (EPI == EPI_DOWN && g.sorted != nullptr) {
        dest = g.sorted[q];
        if (dest < 0 || dest >= g.P) dest = -1;
      }
      if (EPI == EPI_DOWN && g.pair_w != nullptr && dest >= 0) wgt = g.pair_w[dest];
    }
    row_dest[rr] = dest;
    row_w[rr] = wgt;
  }

  const __amdgpu_buffer_rsrc_t ra_rsrc =
      make_rsrc(g.A, (uint32_t)g.a_rows * (uint32_t)g.kdim * 2u);
  const __amdgpu_buffer_rsrc_t rb_rsrc =
      make_rsrc(reinterpret_cast<const unsigned char*>(g.B) + (size_t)e * g.b_bytes, g.b_bytes);
  uint32_t va[A_CH], vb[B_CH];  // per-thread byte offsets (k = 0)
  int sa[A_CH], sb[B_CH];       // LDS element offsets
  int ca[A_CH], cb[B_CH];       // k offset (elements) of the chunk within the step
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int ci = tid + NT * i, r = ci / CPR, c = ci % CPR;
    const uint32_t ro = (r < rows) ? a_row_off(g, row0 + r) : kOob;
    va[i] = ro + c * 16;
    sa[i] = r * LD + c * 8;
    ca[i] = c * 8;
  }
  // B (packed weights): consecutive threads take consecutive 16-byte chunks
  // of one packed block (block bi: tile rows [16 (bi / KBS), +16), k block
  // bi % KBS of the step; chunk q: k chunk q / 16 of row q % 16)
  constexpr int KBS = BK / 32;
  static_assert(BK % 32 == 0, "packed k blocks per step");
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int ci = tid + NT * i, bi = ci / 64, q = ci % 64;
    const int tb = bi / KBS, kb = bi % KBS;
    const int r = tb * 16 + (q & 15), c = kb * 4 + (q >> 4);  // tile row, 16-byte k chunk
    int colb, f = 0;  // packed column block and gate / up half
    if (EPI == EPI_GATEUP) {
      // wave column wn owns TN weight rows: fragment pairs (gate, up) of
      // 32 output columns each
      const int br = tb * 16;
      const int wn = br / TN, fl = (br % TN) >> 5, j = br & 31;
      colb = (n0 + wn * (TN / 2) + (fl >> 1) * 32 + j) / 16;
      f = fl & 1;
    } else {
      colb = (n0 + tb * 16) / 16;
    }
    const uint32_t o = b_block_off<EPI>(g, colb, f);
    vb[i] = (o == kOob) ? kOob : o + (uint32_t)kb * kb_stride<EPI>() + q * 16;
    sb[i] = r * LD + c * 8;
    cb[i] = c * 8;
  }

  // PF register stages: the loads of k step t + PF are issued while step t
  // is multiplied
  bf16x8_t ra[PF][A_CH], rb[PF][B_CH];
  auto gload = [&](int st, int k0) {
    const uint32_t soff = (uint32_t)k0 * 2u;
    const uint32_t soff_b = (uint32_t)(k0 / 32) * kb_stride<EPI>();
    if (k0 + BK <= g.kdim) {
#pragma unroll
      for (int i = 0; i < A_CH; ++i) ra[st][i] = bload8(ra_rsrc, va[i], soff);
#pragma unroll
      for (int i = 0; i < B_CH; ++i) rb[st][i] = bload8(rb_rsrc, vb[i], soff_b);
    } else {  // last, partial k step: chunks at or past kdim read as zero
#pragma unroll
      for (int i = 0; i < A_CH; ++i)
        ra[st][i] = bload8(ra_rsrc, (k0 + ca[i] < g.kdim) ? va[i] : kOob, soff);
#pragma unroll
      for (int i = 0; i < B_CH; ++i)
        rb[st][i] = bload8(rb_rsrc, (k0 + cb[i] < g.kdim) ? vb[i] : kOob, soff_b);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) *reinterpret_cast<bf16x8_t*>(&As[sa[i]]) = ra[st][i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) *reinterpret_cast<bf16x8_t*>(&Bs[sb[i]]) = rb[st][i];
  };

  const int wm = wave % WM, wn = wave / WM;
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  const int nk = (g.kdim + BK - 1) / BK;
  const int r32 = lane & 31;
  const int kh = (lane >> 5) * 8;
  const uint16_t* a_base = &As[(wm * TM + r32) * LD + kh];
  const uint16_t* b_base = &Bs[(wn * TN + r32) * LD + kh];
  auto compute = [&]() {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(a_base + i * 32 * LD + kk * 16);
#pragma unroll
      for (int f = 0; f < FN; ++f)
        b[f] = *reinterpret_cast<const bf16x8_t*>(b_base + f * 32 * LD + kk * 16);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int f = 0; f < FN; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[f], acc[i][f], 0, 0, 0);
    }
  };
#pragma unroll
  for (int st = 0; st < PF; ++st)
    if (st < nk) gload(st, st * BK);
  // the loop body is unrolled PF times so the register stage index is constant
  for (int kt = 0; kt < nk; kt += PF) {
#pragma unroll
    for (int st = 0; st < PF; ++st) {
      if (kt + st < nk) {
        __syncthreads();
        sstore(st);
        __syncthreads();
        if (kt + st + PF < nk) gload(st, (kt + st + PF) * BK);
        compute();
      }
    }
  }

  // Epilogue. C layout of 32x32: element r of lane l is row (r/4)*8 +
  // (l/32)*4 + r%4, column l%32 of the fragment. Each lane turns its values
  // into bf16 outputs (gate-up: bf16(silu(bf16 g) * bf16 u); down: bf16(acc *
  // w[p])) and writes them into the LDS tile; then every thread copies 16-byte
  // row segments to their output rows.
  constexpr int PR = BM / NP;  // rows per pass
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    __syncthreads();  // operand buffers / previous pass no longer read
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = wm * TM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (rr / PR != pass) continue;
        uint16_t* crow = smem + (rr - pass * PR) * CLD;
        if (EPI == EPI_GATEUP) {
#pragma unroll
          for (int pp = 0; pp < FN / 2; ++pp) {
#pragma clang fp contract(off)
            const float gb = round_bf16(acc[i][2 * pp][r]);  // N1
            const float ub = round_bf16(acc[i][2 * pp + 1][r]);
            crow[wn * (TN / 2) + pp * 32 + r32] = (uint16_t)f32_to_bf16(silu_cw(gb) * ub);
          }
        } else {
          const float w = row_w[rr];
#pragma unroll
          for (int f = 0; f < FN; ++f) {
#pragma clang fp contract(off)
            float y = acc[i][f][r];
            if (g.pair_w != nullptr) y = y * w;  // N2: weight on the accumulator
            crow[wn * TN + f * 32 + r32] = (uint16_t)f32_to_bf16(y);
          }
        }
      }
    }
    __syncthreads();
    constexpr int CH = OUT_COLS / 8;  // 16-byte chunks per row
    for (int idx = tid; idx < PR * CH; idx += NT) {
      const int lr = idx / CH, c8 = (idx - lr * CH) * 8;
      const int rr = pass * PR + lr;
      const int dest = row_dest[rr];
      const int col = n0 + c8;
      if (dest < 0 || col >= g.n_out) continue;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + lr * CLD + c8);
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(g.out) + (size_t)dest * g.n_out +
                                  col) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// tiled_dma_kernel: BM x BN block tile (BN weight rows), WM x WN waves, k step
// BK (64 or 32), NS-slot LDS ring filled by direct-to-LDS buffer loads
// (buffer_load_dwordx4 ... lds: lane l's 16 bytes land at M0 + 16*l; an
// out-of-range offset writes zeros). Stages s+1 .. s+NS-1 are loading while
// stage s is multiplied, with no register staging (NS = 2 measured best: a
// 4-slot ring of 32-wide stages ran 1-5 % slower); the MFMA operands of the next 16-wide
// k step are read from LDS while the current step's MFMAs run, and the one
// barrier per stage sits before the last k step of the stage, so the reads of
// the next stage's first step overlap that step's MFMAs. A (activation rows):
// LDS rows of 2*BK bytes, unpadded; 16-byte chunk c of tile row r sits in
// slot c ^ ((r >> 1) & (BK/8 - 1)), which keeps the 16-byte fragment reads of
// 8 consecutive rows on distinct banks. B (packed weights): the packed 1 KiB
// blocks as they come, where a fragment read of 16 rows is 256 contiguous
// bytes.
//
// The 32-row fragments of a tile are dealt to the WM row waves in turn
// (fragment i of wave wm holds rows (i*WM + wm)*32 ..), so a partial tile
// (an expert's last) keeps its rows spread over the waves, and each wave
// runs a copy of the k loop compiled for its count of fragments holding
// rows: fragments wholly past the last row cost no LDS read and no MFMA.
//
// The loads are issued from inline assembly and the waits are explicit
// (s_waitcnt vmcnt(N) lgkmcnt(0); s_barrier): the compiler cannot tell which
// ring slot a direct-to-LDS load writes and would otherwise wait for every
// load in flight before each barrier.
// ---------------------------------------------------------------------------
template <int EPI, int BM, int BN, int WM, int WN, int GM = 0, int BK = 64, int NS = 2>
__global__ __launch_bounds__(64 * WM * WN) void tiled_dma_kernel(GemmArgs g) {
  constexpr int NW = WM * WN;
  constexpr int NT = 64 * NW;
  constexpr int TM = BM / WM, TN = BN / WN;    // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;    // 32x32 fragments per wave
  constexpr int ROWB = BK * 2;                 // bytes per tile row
  constexpr int CPR = BK / 8;                  // 16-byte chunks per row
  constexpr int RPL = 1024 / ROWB;             // rows per 1 KiB load
  constexpr int STAGE = (BM + BN) * ROWB;      // bytes per ring slot
  constexpr int IPW = (BM + BN) / RPL / NW;    // 1 KiB loads per wave per stage
  constexpr int OUT_COLS = (EPI == EPI_GATEUP) ? BN / 2 : BN;
  constexpr int CLD = OUT_COLS + 8;            // output staging row (elements)
  static_assert(BK == 64 || BK == 32, "k step");
  static_assert(NS == 2, "two ring slots");
  static_assert(IPW * RPL * NW == BM + BN, "loads per wave");
  static_assert(BM % 16 == 0 && BN % 16 == 0, "swizzle period");
  static_assert(EPI != EPI_GATEUP || FN % 2 == 0, "gate-up pairs fragments");
  static_assert(EPI != EPI_F32, "logits use the streaming kernel");
  // the bf16 output tile goes through the ring in NP passes of BM / NP rows
  constexpr int NP = (BM * CLD * 2 <= NS * STAGE) ? 1 : 2;
  static_assert((BM / NP) * CLD * 2 <= NS * STAGE && BM % (32 * NP) == 0, "output staging");
  // Gate-up: the one stage issued past the end of k brings the SiLU table
  // (silu_table.h) into its ring slot instead of zeros, into the first 32 KiB
  // of slot 0 or the last 32 KiB of slot 1; the output staging then takes the
  // other end of the ring.
  constexpr bool TAB = EPI == EPI_GATEUP;
  static_assert(!TAB || (NS == 2 && NP == 1 && STAGE >= kSiluTabBytes &&
                         BM * CLD * 2 + kSiluTabBytes <= NS * STAGE &&
                         (NS * STAGE - BM * CLD * 2) % 16 == 0 && kSiluTabBytes % (1024 * NW / 2) == 0),
                "SiLU table space");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NS * STAGE];
  __shared__ int row_dest[BM];
  __shared__ float row_w[BM];
  __shared__ uint32_t row_a[BM];  // byte offset of each tile row's A row (kOob: none)
  __shared__ int tile_info[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0) {
    // XCD-aware block order: the hardware deals workgroup b to XCD b mod 8,
    // so within each run of 8 * XC workgroups XCD x takes logical blocks
    // [x * XC, (x + 1) * XC): 32 consecutive blocks (4 row tiles x 8 column
    // blocks of one expert) share that XCD's L2 (skewed gate-up -1 %, down
    // -2 %, prefill down -5 %; reads past L2 -35 %). A last, incomplete run
    // keeps the hardware order.
    constexpr int XC = 32;
    int L = blockIdx.x;
    {
      const int b = blockIdx.x, x = b & 7, i = b >> 3, run = i / XC;
      if ((run + 1) * 8 * XC <= (int)gridDim.x) L = run * 8 * XC + x * XC + (i - run * XC);
    }
    int e = 0, row0 = 0, rows = 0, nb = 0;
    bool ok;
    if (GM > 0) {
      ok = find_block(g, BM, GM, L, e, row0, rows, nb);
    } else {
      const int slot = L / g.nblk;
      nb = L - slot * g.nblk;
      ok = find_tile(g, BM, slot, e, row0, rows);
    }
    if (!ok) rows = 0;
    if (lane == 0) {
      tile_info[0] = e;
      tile_info[1] = row0;
      tile_info[2] = rows;
      tile_info[3] = nb;
    }
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(tile_info[0]);
  const int row0 = __builtin_amdgcn_readfirstlane(tile_info[1]);
  const int rows = __builtin_amdgcn_readfirstlane(tile_info[2]);
  const int nb = __builtin_amdgcn_readfirstlane(tile_info[3]);
  if (rows <= 0) return;
  const int n0 = nb * OUT_COLS;
  // Row tables, one tile row per thread: output row and weight for the
  // epilogue, and the A row offset that the producers' loads use (for the
  // gate-up a gather through the sorted pairs: one load per row here instead
  // of one per row and producer lane).
  for (int rr = tid; rr < BM; rr += NT) {
    int dest = -1;
    float wgt = 1.0f;
    uint32_t ao = kOob;
    if (rr < rows) {
      const int q = row0 + rr;
      dest = q;
      if (EPI == EPI_DOWN && g.sorted != nullptr) {
        dest = g.sorted[q];
        if (dest < 0 || dest >= g.P) dest = -1;
      }
      if (EPI == EPI_DOWN && g.pair_w != nullptr && dest >= 0) wgt = g.pair_w[dest];
      ao = a_row_off(g, q);
    }
    row_dest[rr] = dest;
    row_w[rr] = wgt;
    row_a[rr] = ao;
  }
  __syncthreads();

  const i32x4_t rsrc_a = raw_rsrc(g.A, (uint32_t)g.a_rows * (uint32_t)g.kdim * 2u);
  const i32x4_t rsrc_b =
      raw_rsrc(reinterpret_cast<const unsigned char*>(g.B) + (size_t)e * g.b_bytes, g.b_bytes);
  // Producer waves: the first NW/2 waves (one per SIMD: wave w runs on SIMD
  // w mod 4) issue every direct load of a stage and the other NW/2 none, so
  // that on each SIMD one wave keeps issuing MFMAs while the other waits for
  // load issue slots (skewed gate-up 1,615-1,631 -> 1,579-1,592 us, down
  // -1 %). A: producer load j fills tile rows [RPL*(j*NPW + wave), +RPL) of a
  // ring slot; lane l writes slot (l%CPR) of row l/CPR, i.e. logical chunk
  // (l%CPR) ^ swz(row). B (packed weights): producer load jb copies packed
  // block jb*NPW + wave, tile rows [16 (b / KBS), +16) at k block b % KBS;
  // its offset is uniform, so it goes in the SGPR offset and every lane's
  // VGPR offset is just 16 * lane.
  constexpr int KBS = BK / 32;  // packed k blocks per stage
  constexpr int NPW = NW / 2;
  constexpr int APP = (BM / RPL) / NPW;             // A loads per producer
  constexpr int BPP = (BN * 2 * BK / 1024) / NPW;   // B loads per producer
  static_assert((BM / RPL) % NPW == 0 && (BN * 2 * BK / 1024) % NPW == 0, "producer loads");
  uint32_t vA[APP];
  uint32_t sB[BPP];
  const uint32_t lane16 = (uint32_t)lane * 16u;
  if (wave < NPW) {
#pragma unroll
    for (int j = 0; j < APP; ++j) {
      const int blk = j * NPW + wave;
      const int r = blk * RPL + lane / CPR;
      const int c = (lane % CPR) ^ ((r >> 1) & (CPR - 1));
      vA[j] = row_a[r] + c * 16;
    }
#pragma unroll
    for (int jb = 0; jb < BPP; ++jb) {
      const int bl = jb * NPW + wave;
      const int tb = bl / KBS, kb = bl % KBS;
      const int br = tb * 16;  // first tile row of the block
      int cb, f = 0;
      if (EPI == EPI_GATEUP) {
        const int wn = br / TN, fl = (br % TN) >> 5, jj = br & 31;
        cb = (n0 + wn * (TN / 2) + (fl >> 1) * 32 + jj) / 16;
        f = fl & 1;
      } else {
        cb = (n0 + br) / 16;
      }
      const uint32_t o = b_block_off<EPI>(g, cb, f);
      sB[jb] = __builtin_amdgcn_readfirstlane((o == kOob) ? kOob : o + (uint32_t)kb * kb_stride<EPI>());
    }
  } else {
#pragma unroll
    for (int j = 0; j < APP; ++j) vA[j] = kOob;
#pragma unroll
    for (int jb = 0; jb < BPP; ++jb) sB[jb] = kOob;
  }
  const uint32_t ring_base = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  const uint32_t wave_lds = ring_base + (uint32_t)wave * 1024u;
  const i32x4_t rsrc_t = raw_rsrc(&kSiluTable, kSiluTabBytes);
  // always inlined: an outlined copy would take its captures through memory
  // and could not hand the descriptors to the loads in SGPRs
  auto issue = [&](int slot, int k0) __attribute__((always_inline)) {
    if (wave >= NPW) return;
    if constexpr (TAB) {
      if (k0 >= g.kdim) {  // past the end of k: the SiLU table, 1 KiB per load
        const uint32_t tb = ring_base + (slot == 0 ? 0u : (uint32_t)(NS * STAGE - kSiluTabBytes));
#pragma unroll
        for (int j = 0; j < kSiluTabBytes / 1024 / NPW; ++j) {
          const uint32_t blk = (uint32_t)(j * NPW + wave) * 1024u;
          dma16(rsrc_t, tb + blk, lane16, blk);
        }
        return;
      }
    }
    const uint32_t soff_a = (uint32_t)k0 * 2u;
    const uint32_t soff_b = (uint32_t)(k0 / 32) * kb_stride<EPI>();
    const uint32_t base = wave_lds + (uint32_t)slot * STAGE;
    if (k0 + BK <= g.kdim) {
#pragma unroll
      for (int j = 0; j < APP; ++j) dma16(rsrc_a, base + j * NPW * 1024, vA[j], soff_a);
#pragma unroll
      for (int jb = 0; jb < BPP; ++jb)
        dma16(rsrc_b, base + (BM / RPL + jb * NPW) * 1024, sB[jb] == kOob ? kOob : lane16,
              __builtin_amdgcn_readfirstlane(sB[jb] == kOob ? 0u : sB[jb] + soff_b));
    } else {  // the k tail: chunks at or past kdim read as zero
#pragma unroll
      for (int j = 0; j < APP; ++j) {
        const int blk = j * NPW + wave;
        const int r = blk * RPL + lane / CPR;
        const int ck = ((lane % CPR) ^ ((r >> 1) & (CPR - 1))) * 8;
        dma16(rsrc_a, base + j * NPW * 1024, (k0 + ck < g.kdim) ? vA[j] : kOob, soff_a);
      }
#pragma unroll
      for (int jb = 0; jb < BPP; ++jb) {
        const int kb = (jb * NPW + wave) % KBS;
        const int ck = kb * 32 + (lane >> 4) * 8;
        const uint32_t vo = (sB[jb] == kOob || k0 + ck >= g.kdim) ? kOob : sB[jb] + lane16;
        dma16(rsrc_b, base + (BM / RPL + jb * NPW) * 1024, vo, soff_b);
      }
    }
  };
  const int wm = wave % WM, wn = wave / WM;
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;
  // Fragment byte offsets inside a ring slot, per k16 step kk, of the wave's
  // first A and first B fragment. Fragment i of A lies i * AFS bytes further
  // (its rows (i*WM + wm)*32 + r32 differ from the first's by a multiple of
  // 32, which leaves the swizzle bits, 1..3 of the row, unchanged) and
  // fragment f of B f * BFS further (16-row blocks 2f on), so the other
  // fragments' offsets are instruction immediates, not registers.
  const int r32 = lane & 31;
  const int khalf = lane >> 5;
  constexpr uint32_t AFS = WM * 32 * ROWB, BFS = 2 * KBS * 1024;
  uint32_t aoff[BK / 16], boff[BK / 16];
  {
    const int r = wm * 32 + r32;
    const int tb = (wn * TN + r32) >> 4, rr = r32 & 15;  // B: tile row wn*TN + r32
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      aoff[kk] = r * ROWB + (((kk * 2 + khalf) ^ ((r >> 1) & (CPR - 1))) * 16);
      const int kb = kk >> 1, c = (kk & 1) * 2 + khalf;
      boff[kk] = BM * ROWB + (tb * KBS + kb) * 1024 + (c * 16 + rr) * 16;
    }
  }
  // MFMA operands of one 16-wide k step, double-buffered across steps. Only
  // the first NVA row fragments of the wave hold tile rows (NVA is a
  // compile-time count, so every variant of the loop is straight-line code).
  constexpr int KK = BK / 16;
  bf16x8_t fa[2][FM], fb[2][FN];
  auto read_step = [&](auto nva_c, int buf, int slot, int kk) {
    constexpr int NVA = decltype(nva_c)::value;
    const unsigned char* sb = ring + slot * STAGE;
#pragma unroll
    for (int i = 0; i < NVA; ++i)
      fa[buf][i] = *reinterpret_cast<const bf16x8_t*>(sb + aoff[kk] + i * AFS);
#pragma unroll
    for (int f = 0; f < FN; ++f)
      fb[buf][f] = *reinterpret_cast<const bf16x8_t*>(sb + boff[kk] + f * BFS);
  };
  auto mfma_step = [&](auto nva_c, int buf) {
    constexpr int NVA = decltype(nva_c)::value;
#pragma unroll
    for (int i = 0; i < NVA; ++i)
#pragma unroll
      for (int f = 0; f < FN; ++f)
        acc[i][f] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][f], acc[i][f], 0, 0, 0);
  };

  const int nk = (g.kdim + BK - 1) / BK;
  // The ring holds stages kt and kt+1 while stage kt is multiplied; each
  // stage ends with vmcnt(0) and a barrier, after which stage kt+2 goes into
  // the slot just read. The one stage issued past the end of k loads the
  // SiLU table into its free slot (gate-up) or zeros (down).
  auto main_loop = [&](auto nva_c) {
    constexpr int NVA = decltype(nva_c)::value;
    // Stage 0 goes out alone and is waited for; stage 1 (or the SiLU table)
    // is issued once the first k step's operands are being read, so that the
    // producers' issue of it overlaps the other waves' first MFMAs.
    issue(0, 0);
    wait_barrier<0>();
    if (NVA > 0) read_step(nva_c, 0, 0, 0);
    issue(1, BK);
    int cur = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const int nxt = (cur + 1 == NS) ? 0 : cur + 1;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int b = kk & 1;
        if (kk + 1 < KK) {
          if (NVA > 0) read_step(nva_c, b ^ 1, cur, kk + 1);
        } else if (kt + 1 < nk) {
          // Stage kt+1 has landed (this wave's loads: the vmcnt; the others':
          // the barrier), and every wave has finished its LDS reads of stage
          // kt (lgkmcnt(0) before the barrier), so its slot takes stage
          // kt+NS.
          static_assert(NS == 2, "per-stage wait for two ring slots");
          wait_barrier<0>();
          issue(cur, (kt + NS) * BK);
          if (NVA > 0) read_step(nva_c, b ^ 1, nxt, 0);
        }
        if (NVA > 0) {
          mfma_step(nva_c, b);
          // schedule: each MFMA followed by one LDS read of the next step,
          // so the reads hide behind the MFMAs instead of bunching before
          // them
#pragma unroll
          for (int q = 0; q < NVA * FN; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (q < NVA + FN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          }
        }
      }
      cur = nxt;
    }
  };
  // row fragment i of wave wm covers tile rows (i * WM + wm) * 32 + [0, 32)
  const int frags = (rows + 31) / 32;
  const int nva = min(FM, max(0, (frags - wm + WM - 1) / WM));
  static_assert(FM <= 5, "main loop variants");
  switch (nva) {
    case 0: main_loop(std::integral_constant<int, 0>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (FM >= 2) main_loop(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (FM >= 3) main_loop(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr (FM >= 4) main_loop(std::integral_constant<int, 4>{}); break;
    default: if constexpr (FM >= 5) main_loop(std::integral_constant<int, FM>{}); break;
  }
  wait_barrier<0>();  // ring free for the output staging; the table landed

  // Epilogue (as in tiled_kernel): bf16 results into LDS, then 16-byte row
  // segments to the output rows, in NP passes of PR rows. The table's slot is
  // that of stage max(nk, 1), the last one issued.
  const bool tab0 = ((nk >= 2 ? nk : 1) & 1) == 0;
  uint16_t* smem =
      reinterpret_cast<uint16_t*>(ring + ((TAB && tab0) ? NS * STAGE - BM * CLD * 2 : 0));
  const float* tab = reinterpret_cast<const float*>(ring + (tab0 ? 0 : NS * STAGE - kSiluTabBytes));
  constexpr int PR = BM / NP;
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
  if (pass > 0) __syncthreads();  // the previous pass's rows are out
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (((i * WM + wm) * 32) / PR != pass) continue;  // fragment rows lie in one pass
    if (i >= nva) continue;  // wholly past the tile's last row: nothing to store
    // accumulator entries r and r + 1 of a lane are rows rr and rr + 1 of one
    // column: each pair becomes bf16 in one conversion
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int rr = (i * WM + wm) * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      uint16_t* crow = smem + (rr - pass * PR) * CLD;
      if (EPI == EPI_GATEUP) {
#pragma unroll
        for (int pp = 0; pp < FN / 2; ++pp) {
#pragma clang fp contract(off)
          // N1: gate and up narrowed to bf16 before the activation
          const uint32_t gu0 = bf16x2_bits(acc[i][2 * pp][r], acc[i][2 * pp + 1][r]);
          const uint32_t gu1 = bf16x2_bits(acc[i][2 * pp][r + 1], acc[i][2 * pp + 1][r + 1]);
          const float y0 = silu_bf16(gu0 & 0xFFFFu, tab) * __uint_as_float(gu0 & 0xFFFF0000u);
          const float y1 = silu_bf16(gu1 & 0xFFFFu, tab) * __uint_as_float(gu1 & 0xFFFF0000u);
          const uint32_t o = bf16x2_bits(y0, y1);
          crow[wn * (TN / 2) + pp * 32 + r32] = (uint16_t)o;
          crow[CLD + wn * (TN / 2) + pp * 32 + r32] = (uint16_t)(o >> 16);
        }
      } else {
        // N2: the weight on the accumulator (row_w is 1 without weights, and
        // y * 1 is y)
        const float w0 = row_w[rr], w1 = row_w[rr + 1];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
#pragma clang fp contract(off)
          const uint32_t o = bf16x2_bits(acc[i][f][r] * w0, acc[i][f][r + 1] * w1);
          crow[wn * TN + f * 32 + r32] = (uint16_t)o;
          crow[CLD + wn * TN + f * 32 + r32] = (uint16_t)(o >> 16);
        }
      }
    }
  }
  __syncthreads();
  constexpr int CH = OUT_COLS / 8;
  for (int idx = tid; idx < PR * CH; idx += NT) {
    const int lr = idx / CH, c8 = (idx - lr * CH) * 8;
    const int dest = row_dest[pass * PR + lr];
    const int col = n0 + c8;
    if (dest < 0 || col >= g.n_out) continue;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + lr * CLD + c8);
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(g.out) + (size_t)dest * g.n_out + col) =
        v;
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

// Grid of slots x nblk workgroups. Consecutive workgroups take adjacent
// column blocks of one expert, i.e. adjacent weight rows (the direct-load tile
// kernel regroups them by XCD itself).
static inline unsigned grid_for(const GemmArgs& g) {
  return (unsigned)((long long)g.slots * g.nblk);
}

// Optional kernel timing, armed per host thread by set_gemm_timing: the next
// GEMM launch goes through hipExtLaunchKernel, which records the kernel's own
// start and end into the two events (no extra packets in the queue), and
// disarms it.
static thread_local hipEvent_t t_start = nullptr;
static thread_local hipEvent_t t_stop = nullptr;

void set_gemm_timing(hipEvent_t start, hipEvent_t stop) {
  t_start = start;
  t_stop = stop;
}

hipError_t timed_launch(const void* kernel, dim3 grid, dim3 block, void** args, hipStream_t s,
                        size_t shm) {
  if (t_start != nullptr && t_stop != nullptr) {
    const hipEvent_t a = t_start, b = t_stop;
    t_start = t_stop = nullptr;
    return hipExtLaunchKernel(kernel, grid, block, args, shm, s, a, b, 0);
  }
  return hipLaunchKernel(kernel, grid, block, args, shm, s);
}

template <typename Kernel>
static hipError_t run(Kernel kernel, unsigned grid, unsigned block, hipStream_t s, GemmArgs& g) {
  if (t_start != nullptr && t_stop != nullptr) {
    const hipEvent_t a = t_start, b = t_stop;
    t_start = t_stop = nullptr;
    void* args[] = {&g};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block), args,
                              0, s, a, b, 0);
  }
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, s, g);
  return hipGetLastError();
}

// Kernel shapes were chosen by measurement on MI355X at the five workload
// shapes (decode 32 tokens / 128 experts, prefill 4096 tokens, 256 experts with
// 16 rows each, a 512-row dense shared expert, skewed 8192 tokens).
template <int EPI>
static hipError_t dispatch(GemmArgs g, hipStream_t s) {
  const bool grouped = g.offsets != nullptr;
  if constexpr (EPI == EPI_F32) {
    // logits: 128 or fewer columns, long k
    if (g.P <= 64) {
      // a few tokens: 16 rows x 16 columns per workgroup, k split over 8 waves
      g.nblk = (g.n_out + 15) / 16;
      g.slots = slots_for(g.P, g.E, 16, false);
      return run(stream_kernel<EPI, 1, 1, 8, 4>, grid_for(g), 512, s, g);
    }
    // many tokens (shapes from sweeps at 512, 4096 and 8192 tokens): up to
    // 1024 tokens 16 rows x 32 columns with k over 8 waves (512 x 2048 x 256:
    // 9.9 -> 7.8 us against 32 x 32); from 8192 tokens 64 rows x 64 columns
    // with k over 8 waves (8192 x 4096 x 128: 39.8 -> 36.5 us against 4
    // waves); between them 32 rows x 64 columns with k over 4 waves
    if (g.P <= 1024) {
      g.nblk = (g.n_out + 31) / 32;
      g.slots = slots_for(g.P, g.E, 16, false);
      return run(stream_kernel<EPI, 1, 2, 8, 4>, grid_for(g), 512, s, g);
    }
    if (g.P >= 8192) {
      g.nblk = (g.n_out + 63) / 64;
      g.slots = slots_for(g.P, g.E, 64, false);
      return run(stream_kernel<EPI, 4, 4, 8, 2>, grid_for(g), 512, s, g);
    }
    g.nblk = (g.n_out + 63) / 64;
    g.slots = slots_for(g.P, g.E, 32, false);
    return run(stream_kernel<EPI, 2, 4, 4, 2>, grid_for(g), 256, s, g);
  } else {
    const double avg_rows = grouped ? (double)g.P / (double)g.E : (double)g.P;
    // LDS tiles pay off with hundreds of rows per expert, from a modest
    // number of tiles on: at 16 experts with 4,000 to 9,000 pairs (one
    // owner's share when 128 experts are split over 8 GPUs) they beat the
    // streaming kernels from 32 nominal tiles on for gate-up (613 -> 308 us
    // at 9,058 pairs of the skewed router, 88 -> 57 us at 4,032 prefill
    // pairs) and from 256 on for down (60 -> 30 us at 4,032 prefill pairs);
    // a 512-row dense expert still streams.
    const int tbm = (EPI == EPI_GATEUP) ? 256 : 128;
    const long long tiled_blocks = (long long)(g.P / tbm) * ((g.n_out + 127) / 128);
    if (avg_rows <= 24.0 || tiled_blocks < (EPI == EPI_GATEUP ? 32 : 256)) {
      if (avg_rows <= 8.0) {
        // decode-like: 16-row tiles of 16 columns; gate-up (gate + up
        // fragments) splits k over 8 waves with 4 k steps in flight per
        // wave, down splits k over 3 waves with 4 in flight
        g.slots = slots_for(g.P, g.E, 16, grouped);
        g.nblk = (g.n_out + 15) / 16;
        if constexpr (EPI == EPI_GATEUP)
          return grouped ? run(stream_kernel<EPI, 1, 1, 8, 4, true>, grid_for(g), 512, s, g)
                         : run(stream_kernel<EPI, 1, 1, 8, 4>, grid_for(g), 512, s, g);
        else
          return grouped ? run(stream_kernel<EPI, 1, 1, 3, 4, true>, grid_for(g), 192, s, g)
                         : run(stream_kernel<EPI, 1, 1, 3, 4>, grid_for(g), 192, s, g);
      }
      // tens of rows per tile: 32-row tiles; gate-up 32 columns with k over
      // 4 waves, down 64 columns with k in one wave for routed rows (2 for a
      // dense expert), measured at 16 rows per expert (256 experts, 512
      // tokens, top-8): against 8 and 2 k-waves, gate-up 190 -> 184 us and
      // down 112 -> 108 us; 16-row tiles, 64- or 128-column gate-up blocks
      // and 128-column down blocks measured slower
      g.slots = slots_for(g.P, g.E, 32, grouped);
      if constexpr (EPI == EPI_GATEUP) {
        g.nblk = (g.n_out + 31) / 32;
        if (grouped) return run(stream_kernel<EPI, 2, 2, 4, 4, true>, grid_for(g), 256, s, g);
        return run(stream_kernel<EPI, 2, 2, 4, 4>, grid_for(g), 256, s, g);
      } else {
        g.nblk = (g.n_out + 63) / 64;
        return grouped ? run(stream_kernel<EPI, 2, 4, 1, 4, true>, grid_for(g), 64, s, g)
                       : run(stream_kernel<EPI, 2, 4, 2, 4>, grid_for(g), 128, s, g);
      }
    } else if constexpr (EPI == EPI_GATEUP) {
      if ((long long)(g.P / 320) * ((g.n_out + 127) / 128) < 512) {
        // too few 320-row tiles to fill 256 CUs: 128 x 128 tiles (64 act
        // columns), 8 waves of 32 x 64, give 2.5x as many workgroups
        // (prefill share of 16 experts: 88 -> 57 us)
        constexpr int BM = 128, BN = 128;
        g.nblk = (g.n_out + BN / 2 - 1) / (BN / 2);
        g.slots = slots_for(g.P, g.E, BM, grouped);
        return run(tiled_dma_kernel<EPI, BM, BN, 4, 2, 4>, grid_for(g), 512, s, g);
      }
      // 320 x 256 tiles on 8 waves with the direct-to-LDS ring; blocks are
      // numbered expert by expert in groups of 4 row tiles, so a weight tile
      // is reused by 4 consecutive workgroups while it is in L2. 320 rows
      // take a whole expert of the 4096-token prefill shape (205-301 rows)
      // in one tile instead of 1-2 tiles of 256 (416 -> 352 us); the row
      // fragments past a tile's last row are skipped
      constexpr int BM = 320, BN = 256;
      g.nblk = (g.n_out + BN / 2 - 1) / (BN / 2);
      g.slots = slots_for(g.P, g.E, BM, grouped);
      return run(tiled_dma_kernel<EPI, BM, BN, 2, 4, 4>, grid_for(g), 512, s, g);
    } else {
      if ((long long)(g.P / 320) * ((g.n_out + 255) / 256) >= 512) {
        // down with enough 320 x 256 tiles to fill the chip: the gate-up's
        // direct-to-LDS ring kernel, the output tile staged in two passes
        // (skewed 8192-token layer 960 -> 930 us)
        constexpr int BM = 320, BN = 256;
        g.nblk = (g.n_out + BN - 1) / BN;
        g.slots = slots_for(g.P, g.E, BM, grouped);
        return run(tiled_dma_kernel<EPI, BM, BN, 2, 4, 4>, grid_for(g), 512, s, g);
      }
      // fewer (one expert-parallel owner's share): 128 x 128 register-staged
      // tiles, 4 workgroups per CU
      constexpr int BM = 128, BN = 128;
      g.nblk = (g.n_out + BN - 1) / BN;
      g.slots = slots_for(g.P, g.E, BM, grouped);
      return run(tiled_kernel<EPI, BM, BN, 64, 2, 2, 1, 4, 0>, grid_for(g), 256, s, g);
    }
  }
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
  g.b_bytes = (uint32_t)packed_expert_bytes(2 * I, H, true);
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
  g.b_bytes = (uint32_t)packed_expert_bytes(H, I, false);
  g.offsets = offsets;
  g.E = E;
  g.P = P;
  g.kdim = I;
  g.n_out = H;
  g.out = expert_out;
  g.pair_w = pair_w;
  return dispatch<EPI_DOWN>(g, s);
}

// ---------------------------------------------------------------------------
// Decode expert FFN in one launch: gate-up + SiLU-mul, then down with the
// routing weight, with no launch boundary between them. The first g1
// workgroups are the gate-up tiles of the streaming kernel (16 rows x 16
// columns, k over 8 waves); the rest are down tiles over the same 16-row
// slots (16 rows x 64 columns). A down tile needs the whole act rows of its
// slot, written by the slot's gu.nblk gate-up workgroups: each of those,
// once its act stores are complete, adds 1 to ready[slot]; a down workgroup
// polls ready[slot] (relaxed) until it is gu.nblk, then acquires at agent
// scope (dropping any stale cached line) before the barrier that lets its
// waves read act. Workgroups are dispatched in
// index order on every XCD, so all gate-up workgroups are resident or done
// before any down workgroup waits, and gate-up workgroups never wait: every
// wait ends. The wait is bounded all the same (kFusedSpin polls with a
// sleep); one that gives up sets *status = 1, skips its tile, and makes the
// waits of the rest give up at once. The last down workgroup of a slot puts
// ready[slot] and done[slot] back to 0, so the counters are zero again for
// the next launch.
// ---------------------------------------------------------------------------
struct FusedArgs {
  GemmArgs gu, dn;
  int g1;         // gate-up workgroups (blocks [0, g1))
  int* ready;     // [slots] gate-up workgroups finished, per slot
  int* done;      // [slots] down workgroups finished, per slot
  int* status;    // 0 = fine, 1 = a wait gave up (results invalid)
};

constexpr int kFusedKS = 8;
constexpr int kFusedDnNFO = 4;  // down tiles: 16 rows x 64 columns (of 32, 64, 128, 256: fastest)
constexpr unsigned kFusedSpin = 1u << 16;
constexpr int kFusedRed =
    stream_red_floats<EPI_GATEUP, 1, 1, kFusedKS>() > stream_red_floats<EPI_DOWN, 1, kFusedDnNFO, kFusedKS>()
        ? stream_red_floats<EPI_GATEUP, 1, 1, kFusedKS>()
        : stream_red_floats<EPI_DOWN, 1, kFusedDnNFO, kFusedKS>();

__global__ __launch_bounds__(64 * kFusedKS) void fused_ffn_kernel(FusedArgs fa) {
  __shared__ float red[kFusedRed];  // one buffer for either phase
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < fa.g1) {
    const int blk = blockIdx.x;
    // act goes out as agent-scope atomic stores, performed at the device's
    // point of coherence. Each wave then waits for its own stores to
    // complete (the barrier alone does not), so every act store of the tile
    // is done, device-wide, before the count moves. That makes the count a
    // release for these stores without an agent-scope release fence, whose
    // L2 write-back per workgroup measured 2.2x slower for the whole FFN.
    if (!stream_body<EPI_GATEUP, 1, 1, kFusedKS, 4, true, true>(fa.gu, blk, red)) return;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      __hip_atomic_fetch_add(fa.ready + blk / fa.gu.nblk, 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int blk = (int)blockIdx.x - fa.g1;
  const int slot = blk / fa.dn.nblk;
  __shared__ int go;  // 0: no tile, 1: compute, 2: gave up
  if (tid < 64) {
    int e, row0, rows;
    const bool ok = find_tile(fa.dn, 16, slot, e, row0, rows);
    if (tid == 0) {
      int st = ok ? 1 : 0;
      if (ok) {
        // relaxed polls (an acquire load would invalidate the L2 on every
        // poll), one acquire once the count is complete
        unsigned it = 0;
        while (__hip_atomic_load(fa.ready + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
               fa.gu.nblk) {
          if (++it > kFusedSpin ||
              __hip_atomic_load(fa.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
            __hip_atomic_store(fa.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            st = 2;
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
        // a wait that gave up elsewhere leaves every count of this launch in
        // doubt (a late gate-up workgroup may add to a count already reset):
        // give up too
        if (st == 1 &&
            __hip_atomic_load(fa.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
          st = 2;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      go = st;
    }
  }
  __syncthreads();
  const int st = go;
  if (st == 0) return;
  if (st == 1) stream_body<EPI_DOWN, 1, kFusedDnNFO, kFusedKS, 3, false, true>(fa.dn, blk, red);
  __syncthreads();
  if (tid == 0) {
    // a count only (no data is published through it): relaxed; every down
    // workgroup of the slot finished polling ready[slot] before adding here
    const int old =
        __hip_atomic_fetch_add(fa.done + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == fa.dn.nblk - 1) {
      __hip_atomic_store(fa.ready + slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(fa.done + slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

int fused_ffn_workspace_ints(int P, int E, bool grouped) {
  return 2 * slots_for(P, E, 16, grouped) + 1;
}

hipError_t launch_fused_ffn(const uint16_t* x, int T, int H, const uint16_t* w_gu,
                            const uint16_t* w_d, int E, int I, const int32_t* sorted,
                            const int32_t* offsets, int K, const float* pair_w, uint16_t* act,
                            uint16_t* expert_out, int* ws, hipStream_t s) {
  const bool grouped = offsets != nullptr;
  FusedArgs fa{};
  GemmArgs& gu = fa.gu;
  gu.A = x;
  gu.a_rows = T;
  gu.sorted = sorted;
  gu.gather_k = K;
  gu.B = w_gu;
  gu.b_bytes = (uint32_t)packed_expert_bytes(2 * I, H, true);
  gu.offsets = offsets;
  gu.E = E;
  gu.P = T * K;
  gu.kdim = H;
  gu.n_out = I;
  gu.out = act;
  gu.slots = slots_for(gu.P, E, 16, grouped);
  gu.nblk = (I + 15) / 16;
  GemmArgs& dn = fa.dn;
  dn.A = act;
  dn.a_rows = gu.P;
  dn.sorted = sorted;
  dn.gather_k = 0;
  dn.B = w_d;
  dn.b_bytes = (uint32_t)packed_expert_bytes(H, I, false);
  dn.offsets = offsets;
  dn.E = E;
  dn.P = gu.P;
  dn.kdim = I;
  dn.n_out = H;
  dn.out = expert_out;
  dn.pair_w = pair_w;
  dn.slots = gu.slots;
  dn.nblk = (H + 16 * kFusedDnNFO - 1) / (16 * kFusedDnNFO);
  fa.g1 = gu.slots * gu.nblk;
  fa.ready = ws;
  fa.done = ws + gu.slots;
  fa.status = ws + 2 * gu.slots;
  const long long grid = (long long)fa.g1 + (long long)dn.slots * dn.nblk;
  void* args[] = {&fa};
  return timed_launch(reinterpret_cast<const void*>(fused_ffn_kernel), dim3((unsigned)grid),
                      dim3(64 * kFusedKS), args, s);
}

hipError_t launch_logits(const uint16_t* x, int T, int H, const uint16_t* w, int N,
                         const float* bias, float* out, hipStream_t s) {
  GemmArgs g{};
  g.A = x;
  g.a_rows = T;
  g.sorted = nullptr;
  g.gather_k = 0;
  g.B = w;
  g.b_bytes = (uint32_t)((size_t)N * H * 2);
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
