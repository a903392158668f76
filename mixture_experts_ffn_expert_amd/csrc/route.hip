// route.hip -- softmax top-k routing and stable expert grouping on gfx950.
//
// Router: the ungrouped softmax top-k with renormalisation that vllm.cpp
// PR #509 ("MoE combine/gate ops", Honest gaps) names as the covered router
// form. Grouping: the per-expert row grouping the grouped expert GEMMs run
// over (issue #3094 row statement; PR #523 What changed, grouped over expert
// ids).
//
// Kernel 1 (topk_kernel): one wavefront per token. Lane l holds logits
//   e = l + 64*j as order-preserving integer keys. Each of the K rounds takes
//   the wavefront maximum key (DPP reduction) and, by one ballot per j, the
//   lowest expert id holding it, so ties go to the lower id; lane k keeps the
//   k-th logit, computes e_k = exp(l_k - l_0), every lane forms the same
//   sequential f32 sum, lane k divides.
// Grouping (group_kernel for up to 4096 pairs, else the count kernel over
//   1024-pair segments followed by the scan and the scatter, in one launch
//   where the count table is small): (i) per-wave expert histograms in LDS,
//   (ii) an exclusive scan over experts (and segments) gives every wave its
//   first output position per expert, (iii) each wave walks its part in
//   order, 64 pairs at a time, ranks equal experts inside the 64 by ballots,
//   and scatters. No atomic decides an order, so the permutation is the
//   stable one and is reproducible.
#include <mutex>

#include "device_math.h"
#include "launch.h"

// Grouping scratch held by the library for moe_route_noalloc: the
// per-(segment, expert) counts of the segmented grouping, 4 bytes each, at
// most kRouteScratchBytes. Each GPU the library runs on holds its own copy
// until the process ends. Host code never uses this name as an address: it
// takes the device address from hipGetSymbolAddress (route_scratch below).
static __device__ __align__(256) int32_t scratch[moe::kRouteScratchBytes / 4];

namespace moe {

constexpr int kMaxE = 1024;
constexpr int kMaxPerLane = kMaxE / 64;

// Wavefront max of a 32-bit value (ROCm device library, DPP based).
extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);

// Order-preserving map of a non-NaN float to uint32 (larger float, larger
// key). +0 and -0 must be made equal by the caller. Every key is >= 1, so 0
// marks "already taken".
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Inverse of order_key for keys of non-NaN floats.
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Top-K of one token's E logits by one wavefront; lane k < K writes ids[k]
// and w[k]. The selected logit is recovered from its key: it equals the
// logit except that -0 reads as +0, which changes no weight (x - (+-0) and
// (+-0) - (+-0) give the same exp argument up to the sign of zero, and
// exp(+-0) = 1).
template <int NP>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int E, int K,
                                           int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int nper = (E + 63) >> 6;
  uint32_t key[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int e = lane + 64 * j;
    uint32_t kj = 0;
    if (j < nper && e < E) {
      float x = row[e];
      if (x != x) x = -__builtin_inff();  // NaN ranks as -inf
      if (x == 0.0f) x = 0.0f;            // -0 ties with +0
      kj = order_key(x);
    }
    key[j] = kj;
  }
  uint32_t my_key = 0;  // lane k keeps the k-th selected key
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < NP; ++j) m = max(m, key[j]);
    const uint32_t M = __ockl_wfred_max_u32(m);
    // the lowest expert id holding the maximum: lower j first, then lower lane
    int sel = 0;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j >= nper) break;
      const uint64_t hit = __ballot(key[j] == M);
      if (hit) {
        sel = (__ffsll((long long)hit) - 1) + 64 * j;
        break;
      }
    }
#pragma unroll
    for (int j = 0; j < NP; ++j)
      if (sel == lane + 64 * j) key[j] = 0;  // taken
    if (lane == k) {
      my_key = M;
      my_id = sel;
    }
  }
  // renormalised weights: e_k = exp(l_k - l_0), S = ((e_0 + e_1) + ...), w_k = e_k / S
  const float my_val = key_value(my_key);
  const float top = lane_f32(my_val, 0);
  float ek;
  {
#pragma clang fp contract(off)
    const float d = my_val - top;
    ek = exp_cw(d);
  }
  float S = lane_f32(ek, 0);
  for (int k = 1; k < K; ++k) {
#pragma clang fp contract(off)
    S = S + lane_f32(ek, k);
  }
  if (lane < K) {
    ids[lane] = my_id;
    w[lane] = __fdiv_rn(ek, S);
  }
}

template <int NP>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int K, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  topk_token<NP>(logits + (size_t)t * E, E, K, ids + (size_t)t * K, w + (size_t)t * K);
}

// ---------------------------------------------------------------------------
// General router: sigmoid or full-softmax scores, an optional selection bias
// and group-limited selection (the grouped / biased / sigmoid forms that
// issue #3094's row statement and PR #509's Honest gaps list as the router
// gaps left; their arithmetic follows the DeepSeek-V2 / V3 technical
// reports). Per token, in f32, each operation rounded on its own:
//   s_e = sigmoid(l_e), or z_e / S with m = max l, z_e = exp(l_e - m) and S
//       the butterfly sum (lane e%64 adds its z in increasing e, then lanes
//       l and l^m are added for m = 32 .. 1);
//   c_e = s_e (+ bias_e); NaN ranks as -inf;
//   groups of E/n_group consecutive experts scored by their largest c or the
//   sum of their two largest; the topk_group best groups stay allowed (ties
//   to the lower group);
//   K rounds pick the largest allowed c (ties to the lower id);
//   w_k = s_{e_k}, renormalised by the sequential sum over k when asked.
// ---------------------------------------------------------------------------
struct ScoredRouter {
  int sigmoid;          // 1: sigmoid scores, 0: softmax over all E
  const float* bias;    // [E] selection bias or null
  int n_group;          // 1: no group limit
  int topk_group;       // groups kept
  int group_top2;       // 1: group score = sum of its two largest c, 0: largest c
  int renorm;           // 1: renormalise the K weights
};

__device__ __forceinline__ uint32_t select_key(float c) {
  if (c != c) c = -__builtin_inff();  // NaN ranks as -inf
  if (c == 0.0f) c = 0.0f;            // -0 ties with +0
  return order_key(c);
}

template <int NP>
__device__ __forceinline__ void topk_scored_token(const float* __restrict__ row, int E, int K,
                                                  const ScoredRouter& r, uint32_t* gkeys,
                                                  int32_t* __restrict__ ids,
                                                  float* __restrict__ w) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int nper = (E + 63) >> 6;
  float s[NP];
  uint32_t key[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int e = lane + 64 * j;
    float x = -__builtin_inff();
    if (j < nper && e < E) {
      x = row[e];
      if (x != x) x = -__builtin_inff();
    }
    s[j] = x;  // logits for now
  }
  if (r.sigmoid) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j >= nper) break;
      s[j] = sigmoid_cw(s[j]);
    }
  } else {
    uint32_t mk = 0;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j >= nper) break;
      if (lane + 64 * j < E) mk = max(mk, select_key(s[j]));
    }
    const float m = key_value(__ockl_wfred_max_u32(mk));
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j >= nper) break;
      if (lane + 64 * j < E) {
        const float z = exp_cw(s[j] - m);
        s[j] = z;
        p = (j == 0) ? z : p + z;
      }
    }
#pragma unroll
    for (int m2 = 32; m2 >= 1; m2 >>= 1) p = p + __shfl_xor(p, m2);
    const float S = lane_f32(p, 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j >= nper) break;
      if (lane + 64 * j < E) s[j] = __fdiv_rn(s[j], S);
    }
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) key[j] = 0;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    if (j >= nper) break;
    const int e = lane + 64 * j;
    if (e < E) key[j] = select_key(r.bias != nullptr ? s[j] + r.bias[e] : s[j]);
  }

  if (r.n_group > 1) {
    // Group scores: the selection keys go through LDS, and lane g < n_group
    // scans its group's E/n_group keys for the largest two.
    const int gs = E / r.n_group;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j >= nper) break;
      if (lane + 64 * j < E) gkeys[lane + 64 * j] = key[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t gkey = 0;  // lane g holds group g's score key
    if (lane < r.n_group) {
      uint32_t k1 = 0, k2 = 0;  // largest and second largest key of the group
      for (int i = 0; i < gs; ++i) {
        const uint32_t v = gkeys[lane * gs + i];
        if (v > k1) {
          k2 = k1;
          k1 = v;
        } else if (v > k2) {
          k2 = v;
        }
      }
      float score = key_value(k1);
      if (r.group_top2 && gs > 1) score = score + key_value(k2);
      gkey = select_key(score);
    }
    uint64_t keep = 0;
    for (int k = 0; k < r.topk_group; ++k) {
      const uint32_t M = __ockl_wfred_max_u32(gkey);
      const uint64_t hit = __ballot(gkey == M && gkey != 0);
      const int g = __ffsll((long long)hit) - 1;
      keep |= 1ull << g;
      if (lane == g) gkey = 0;
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !((keep >> (e / gs)) & 1ull)) key[j] = 0;
    }
  }

  float my_s = 0.0f;  // lane k keeps the k-th selected score
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < NP; ++j) m = max(m, key[j]);
    const uint32_t M = __ockl_wfred_max_u32(m);
    int sel = 0;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j >= nper) break;
      const uint64_t hit = __ballot(key[j] == M);
      if (hit) {
        sel = (__ffsll((long long)hit) - 1) + 64 * j;
        break;
      }
    }
    float sv = 0.0f;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (sel == lane + 64 * j) key[j] = 0;  // taken
      if (j == (sel >> 6)) sv = s[j];
    }
    const float s_sel = lane_f32(sv, sel & 63);
    if (lane == k) {
      my_s = s_sel;
      my_id = sel;
    }
  }
  float wk = my_s;
  if (r.renorm) {
    float S = lane_f32(my_s, 0);
    for (int k = 1; k < K; ++k) S = S + lane_f32(my_s, k);
    wk = __fdiv_rn(my_s, S);
  }
  if (lane < K) {
    ids[lane] = my_id;
    w[lane] = wk;
  }
}

template <int NP>
__global__ __launch_bounds__(256) void topk_scored_kernel(const float* __restrict__ logits, int T,
                                                          int E, int K, ScoredRouter r,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
  __shared__ uint32_t gkeys[4][kMaxE];  // per wave: selection keys for the group scores
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  topk_scored_token<NP>(logits + (size_t)t * E, E, K, r, gkeys[threadIdx.x >> 6],
                        ids + (size_t)t * K, w + (size_t)t * K);
}

constexpr int kGroupWaves = 8;
// The largest pair count the single-workgroup grouping kernel handles.
constexpr int kGroupSeg = 4096;
// Pairs per workgroup segment of the multi-workgroup grouping above that:
// 1024 pairs keep each wave's in-order walk to two steps of 64 (4096-pair
// segments measured 23 us for the 32768 pairs of the 4096-token prefill
// shape, mostly in the scatter's serial walk).
constexpr int kScatterSeg = 1024;

// Items per lane of a wave's part: a segment of n pairs gives each of the
// kGroupWaves waves a contiguous part of ceil(n / kGroupWaves) pairs, 64 per
// item.
constexpr int kGroupItems = kGroupSeg / kGroupWaves / 64;      // 8
constexpr int kScatterItems = kScatterSeg / kGroupWaves / 64;  // 2
static_assert(kGroupItems * 64 * kGroupWaves == kGroupSeg &&
              kScatterItems * 64 * kGroupWaves == kScatterSeg, "parts of whole items");

// The expert ids of wave w's part [wb, we) of segment [beg, end): item j of
// lane l is pair wb + 64 j + l (-1 past the part). All loads are issued
// before the first is used, and the ids stay in registers for both the count
// and the scatter.
template <int NI>
__device__ __forceinline__ void load_part(const int32_t* ids, int beg, int end, int& wb, int& we,
                                          int (&v)[NI]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seg = (end - beg + kGroupWaves - 1) / kGroupWaves;
  wb = min(end, beg + wave * seg);
  we = min(end, wb + seg);
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int p = wb + 64 * j + lane;
    v[j] = (p < we) ? ids[p] : -1;
  }
}

// Per-wave expert counts of the waves' parts: cur[w][e] for e < E (entries
// past E are not touched). Counts commute, so LDS atomics are fine here.
template <int NI>
__device__ __forceinline__ void count_part(const int (&v)[NI], int E, int (*cur)[kMaxE]) {
  const int wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x)
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) cur[w][e] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NI; ++j)
    if ((unsigned)v[j] < (unsigned)E) atomicAdd(&cur[wave][v[j]], 1);
  __syncthreads();
}

// Stable in-order scatter of the wave's part. cur[w][e] holds, on entry, wave
// w's first output position for expert e; the wave walks its part 64 pairs
// at a time, ranking equal experts inside the 64 with ballots over the id
// bits.
template <int NI>
__device__ __forceinline__ void scatter_part(const int (&v)[NI], int wb, int we, int E,
                                             int (*cur)[kMaxE], int32_t* __restrict__ sorted) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int base = wb + 64 * j;
    if (base >= we) break;  // uniform over the wave
    const int p = base + lane;
    int e = v[j];
    const bool valid = p < we && (unsigned)e < (unsigned)E;  // ids come from the top-k kernels
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t m = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    int pos = 0;
    if (valid) pos = cur[wave][e] + rank;
    __builtin_amdgcn_wave_barrier();
    // the highest lane of each peer group advances the cursor
    if (valid && (peers >> lane) == 1ull) cur[wave][e] = pos + 1;
    __builtin_amdgcn_wave_barrier();
    if (valid) sorted[pos] = p;
  }
}

// Exclusive scan of tot[e] over experts e < E by the whole workgroup: thread
// i owns experts [e0, e1) = [i*per, (i+1)*per) in order and gets the first
// position of expert e0; the next owned expert starts tot[e] later.
__device__ __forceinline__ int scan_experts(int E, const int* tot, int* wave_tot, int& e0,
                                            int& e1) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nthreads = kGroupWaves * 64;
  const int per = (E + nthreads - 1) / nthreads;
  e0 = min(E, tid * per);
  e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += tot[e];
  int incl = local;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m);
    if (lane >= m) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wave_tot[w];
  return run;
}

// Single workgroup (kGroupWaves waves, P <= kGroupSeg): counts, the
// exclusive scan over experts, then the scatter.
__global__ __launch_bounds__(kGroupWaves * 64) void group_kernel(const int32_t* __restrict__ ids,
                                                                 int P, int E,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ sorted) {
  __shared__ int cur[kGroupWaves][kMaxE];  // per-wave counts, then per-wave cursors
  __shared__ int tot[kMaxE];
  __shared__ int wave_tot[kGroupWaves];
  int v[kGroupItems];
  int wb, we;
  load_part(ids, 0, P, wb, we, v);
  count_part(v, E, cur);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) n += cur[w][e];
    tot[e] = n;
  }
  __syncthreads();
  int e0, e1;
  int run = scan_experts(E, tot, wave_tot, e0, e1);
  for (int e = e0; e < e1; ++e) {
    offsets[e] = run;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) {
      const int n = cur[w][e];
      cur[w][e] = run;  // cursor of wave w for expert e
      run += n;
    }
  }
  if (threadIdx.x == 0) offsets[E] = P;
  __syncthreads();
  scatter_part(v, wb, we, E, cur, sorted);
}

// Multi-workgroup grouping, step 1: expert counts of each segment of
// kScatterSeg pairs -> cnt[b][e].
__global__ __launch_bounds__(kGroupWaves * 64) void group_count_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ cnt) {
  __shared__ int cur[kGroupWaves][kMaxE];
  const int beg = blockIdx.x * kScatterSeg;
  const int end = min(P, beg + kScatterSeg);
  int v[kScatterItems];
  int wb, we;
  load_part(ids, beg, end, wb, we, v);
  count_part(v, E, cur);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) n += cur[w][e];
    cnt[(size_t)blockIdx.x * E + e] = n;
  }
}

// Step 2 (one workgroup): expert offsets, and cnt[b][e] replaced by segment
// b's first output position for expert e.
__global__ __launch_bounds__(1024) void group_scan_kernel(int32_t* __restrict__ cnt, int nseg,
                                                          int P, int E,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int wave_tot[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int e = tid;  // E <= 1024: one expert per thread
  // segments are read 16 at a time, all 16 loads in flight before the sums
  constexpr int SB = 16;
  int tot = 0;
  if (e < E)
    for (int b0 = 0; b0 < nseg; b0 += SB) {
      int v[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) v[j] = (b0 + j < nseg) ? cnt[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < SB; ++j) tot += v[j];
    }
  int incl = tot;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m);
    if (lane >= m) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - tot;
  for (int w = 0; w < wave; ++w) run += wave_tot[w];
  if (e < E) {
    offsets[e] = run;
    for (int b0 = 0; b0 < nseg; b0 += SB) {
      int v[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) v[j] = (b0 + j < nseg) ? cnt[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        if (b0 + j < nseg) cnt[(size_t)(b0 + j) * E + e] = run;
        run += v[j];
      }
    }
  }
  if (tid == 0) offsets[E] = P;
}

// Wave cursors from a segment's base positions: on entry cur[w][e] holds
// wave w's count of expert e; on return its first output position, base[e] +
// the counts of the waves before w (in order). base_of(e) gives base[e].
template <typename Base>
__device__ __forceinline__ void wave_cursors(int E, int (*cur)[kMaxE], Base base_of) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = base_of(e);
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) {
      const int n = cur[w][e];
      cur[w][e] = run;
      run += n;
    }
  }
  __syncthreads();
}

// Step 3: each segment scatters its pairs in order from its own positions.
__global__ __launch_bounds__(kGroupWaves * 64) void group_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, const int32_t* __restrict__ base,
    int32_t* __restrict__ sorted) {
  __shared__ int cur[kGroupWaves][kMaxE];
  const int beg = blockIdx.x * kScatterSeg;
  const int end = min(P, beg + kScatterSeg);
  int v[kScatterItems];
  int wb, we;
  load_part(ids, beg, end, wb, we, v);
  count_part(v, E, cur);
  const int32_t* seg_base = base + (size_t)blockIdx.x * E;
  wave_cursors(E, cur, [=](int e) { return seg_base[e]; });
  scatter_part(v, wb, we, E, cur, sorted);
}

// Steps 2 and 3 in one launch, for count tables of at most kFoldCounts
// entries: every segment's workgroup reads the whole table cnt[b][e] (coalesced,
// up to kFoldLoads loads per thread in flight at once), sums each expert's
// total and the counts of the segments before its own, scans the totals, and
// scatters from its own positions; workgroup 0 also writes the offsets. The
// table is only read, so the workgroups do not depend on one another.
constexpr int kFoldLoads = 16;
constexpr int kFoldCounts = kFoldLoads * kGroupWaves * 64 * 2;  // 16,384
__global__ __launch_bounds__(kGroupWaves * 64) void group_scan_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, const int32_t* __restrict__ cnt, int nseg,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted) {
  __shared__ int cur[kGroupWaves][kMaxE];
  __shared__ int tot[kMaxE];
  __shared__ int pre[kMaxE];
  __shared__ int wave_tot[kGroupWaves];
  const int tid = threadIdx.x;
  constexpr int NT = kGroupWaves * 64;
  const int seg = blockIdx.x;
  const int beg = seg * kScatterSeg;
  const int end = min(P, beg + kScatterSeg);
  int v[kScatterItems];
  int wb, we;
  load_part(ids, beg, end, wb, we, v);
  for (int e = tid; e < E; e += NT) {
    tot[e] = 0;
    pre[e] = 0;
  }
  count_part(v, E, cur);  // its barriers also order the zeroing above
  const int n = E * nseg;
  for (int i0 = 0; i0 < n; i0 += NT * kFoldLoads) {
    int c[kFoldLoads];
#pragma unroll
    for (int j = 0; j < kFoldLoads; ++j) {
      const int i = i0 + j * NT + tid;
      c[j] = (i < n) ? cnt[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kFoldLoads; ++j) {
      const int i = i0 + j * NT + tid;
      if (c[j] != 0) {  // i < n
        const int b = i / E, e = i - b * E;
        atomicAdd(&tot[e], c[j]);  // integer sums: the order does not matter
        if (b < seg) atomicAdd(&pre[e], c[j]);
      }
    }
  }
  __syncthreads();
  int e0, e1;
  int run = scan_experts(E, tot, wave_tot, e0, e1);
  for (int e = e0; e < e1; ++e) {
    if (seg == 0) offsets[e] = run;
    pre[e] += run;  // the segment's first position for expert e
    run += tot[e];
  }
  if (seg == 0 && tid == 0) offsets[E] = P;
  __syncthreads();
  wave_cursors(E, cur, [&](int e) { return pre[e]; });
  scatter_part(v, wb, we, E, cur, sorted);
}

size_t route_workspace_bytes(int T, int E, int K) {
  const long long P = (long long)T * K;
  if (P <= kGroupSeg) return 0;
  const long long nseg = (P + kScatterSeg - 1) / kScatterSeg;
  return (size_t)(nseg * E * 4);
}

// Stable grouping of the P = T*K routed pairs by expert.
static hipError_t launch_grouping(const int32_t* ids, int P, int E, int32_t* offsets,
                                  int32_t* sorted, void* ws, hipStream_t s) {
  if (P <= kGroupSeg) {
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kGroupWaves * 64), 0, s, ids, P, E, offsets,
                       sorted);
  } else {
    const int nseg = (P + kScatterSeg - 1) / kScatterSeg;
    int32_t* cnt = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL(group_count_kernel, dim3(nseg), dim3(kGroupWaves * 64), 0, s, ids, P, E,
                       cnt);
    if ((long long)nseg * E <= kFoldCounts) {
      hipLaunchKernelGGL(group_scan_scatter_kernel, dim3(nseg), dim3(kGroupWaves * 64), 0, s, ids,
                         P, E, cnt, nseg, offsets, sorted);
    } else {
      hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, nseg, P, E, offsets);
      hipLaunchKernelGGL(group_scatter_kernel, dim3(nseg), dim3(kGroupWaves * 64), 0, s, ids, P,
                         E, cnt, sorted);
    }
  }
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                        int32_t* offsets, int32_t* sorted, void* ws, hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, logits, T, E, K, ids, w);
  else if (E <= 128)
    hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, logits, T, E, K, ids, w);
  else if (E <= 256)
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, logits, T, E, K, ids, w);
  else
    hipLaunchKernelGGL(topk_kernel<kMaxPerLane>, grid, block, 0, s, logits, T, E, K, ids, w);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_grouping(ids, T * K, E, offsets, sorted, ws, s);
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current and kept.
namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kRouteScratchDevices] = {};
}  // namespace

hipError_t route_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kRouteScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_route_scored(const float* logits, int T, int E, int K, int sigmoid,
                               const float* bias, int n_group, int topk_group, int group_top2,
                               int renorm, int32_t* ids, float* w, int32_t* offsets,
                               int32_t* sorted, void* ws, hipStream_t s) {
  const ScoredRouter r{sigmoid, bias, n_group, topk_group, group_top2, renorm};
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(topk_scored_kernel<1>, grid, block, 0, s, logits, T, E, K, r, ids, w);
  else if (E <= 128)
    hipLaunchKernelGGL(topk_scored_kernel<2>, grid, block, 0, s, logits, T, E, K, r, ids, w);
  else if (E <= 256)
    hipLaunchKernelGGL(topk_scored_kernel<4>, grid, block, 0, s, logits, T, E, K, r, ids, w);
  else
    hipLaunchKernelGGL(topk_scored_kernel<kMaxPerLane>, grid, block, 0, s, logits, T, E, K, r,
                       ids, w);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_grouping(ids, T * K, E, offsets, sorted, ws, s);
}

}  // namespace moe
