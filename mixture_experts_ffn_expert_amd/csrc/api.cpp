// api.cpp -- the C ABI of the MoE expert path (declared in include/moe.h):
// host-side argument validation, refusals with named messages, then one
// stream-ordered launch sequence per call. No allocation, no synchronisation.
//
// Refusal rule: vllm.cpp PR #509 review comment -- only the f32 and bf16
// arms exist, and anything else (f16) is refused with a message that names
// the missing piece instead of being reinterpreted.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = {0};

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_err() { g_err[0] = 0; }

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxDevices = 64;

std::mutex g_dev_mu;
int g_dev_state[kMaxDevices] = {0};  // 0 unknown, 1 gfx950, 2 other

moe_status check_device(const char* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_E_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_E_HIP, "%s: device index %d out of range", fn, dev);
  int st;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    st = g_dev_state[dev];
  }
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(MOE_E_HIP, "%s: hipGetDeviceProperties failed: %s", fn, hipGetErrorString(e));
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    g_dev_state[dev] = st;
    if (st == 2)
      return fail(MOE_E_HIP, "%s: device %d is %s; this library is built for gfx950 (MI355X) only",
                  fn, dev, prop.gcnArchName);
  }
  if (st == 2) return fail(MOE_E_HIP, "%s: device %d is not gfx950 (MI355X)", fn, dev);
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const char* dtype_name(moe_dtype d) {
  switch (d) {
    case MOE_F32: return "f32";
    case MOE_BF16: return "bf16";
    case MOE_F16: return "f16";
  }
  return "unknown";
}

moe_status check_dtype(const char* fn, const char* arg, moe_dtype d) {
  if (d == MOE_F32 || d == MOE_BF16) return MOE_OK;
  return fail(MOE_E_DTYPE, "%s: %s dtype %s unsupported (only the f32 and bf16 arms exist)", fn, arg,
              dtype_name(d));
}

#define REQUIRE_PTR(fn, p)                                                          \
  do {                                                                              \
    if ((p) == nullptr) return fail(MOE_E_INVALID, "%s: %s is NULL", fn, #p);       \
    if (!aligned16(p)) return fail(MOE_E_INVALID, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

#define REQUIRE_NONNULL(fn, p)                                                      \
  do {                                                                              \
    if ((p) == nullptr) return fail(MOE_E_INVALID, "%s: %s is NULL", fn, #p);       \
  } while (0)

moe_status hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(MOE_E_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return MOE_OK;
}

bool fits_i32(long long v) { return v >= 0 && v < (1LL << 31); }

// The GEMM kernels address each operand matrix (and each expert's weight
// block) through a buffer resource of at most 2^31 bytes: 2^30 bf16 values.
bool fits_buf(long long elems) { return elems >= 0 && elems < (1LL << 30); }

// One expert's packed weights are addressed the same way: below 2^31 bytes.
bool fits_packed(int R, int kdim, bool gateup) {
  return moe::packed_expert_bytes(R, kdim, gateup) < (size_t)(1u << 31);
}

// A packed weight descriptor as the grouped GEMMs need it: filled by
// moe_pack_weights (layout tag), of the call's kind and dimensions, with an
// aligned data pointer and the expert size the packed layout implies.
moe_status check_weights(const char* fn, const char* arg, const moe_weights* w,
                         moe_pack_kind kind, int E, int R, int K) {
  if (w == nullptr) return fail(MOE_E_INVALID, "%s: %s is NULL", fn, arg);
  if (w->layout != MOE_WEIGHTS_PACKED_V1)
    return fail(MOE_E_INVALID,
                "%s: %s is not a packed weight descriptor (layout tag 0x%08x); pack the row-major "
                "weights with moe_pack_weights", fn, arg, w->layout);
  const bool gu = kind == MOE_PACK_GATEUP;
  if (w->kind != (int32_t)kind)
    return fail(MOE_E_INVALID, "%s: %s was packed as %s, this call needs %s", fn, arg,
                w->kind == MOE_PACK_GATEUP ? "MOE_PACK_GATEUP" : "MOE_PACK_PLAIN",
                gu ? "MOE_PACK_GATEUP" : "MOE_PACK_PLAIN");
  if (w->E != E || w->R != R || w->K != K)
    return fail(MOE_E_INVALID, "%s: %s holds %d experts of [%d, %d], the call needs %d of [%d, %d]",
                fn, arg, w->E, w->R, w->K, E, R, K);
  if (w->expert_bytes != moe::packed_expert_bytes(R, K, gu))
    return fail(MOE_E_INVALID, "%s: %s expert size %llu bytes does not match the packed layout",
                fn, arg, (unsigned long long)w->expert_bytes);
  if (w->data == nullptr || !aligned16(w->data))
    return fail(MOE_E_INVALID, "%s: %s data is NULL or not 16-byte aligned", fn, arg);
  return MOE_OK;
}

// Timing armed by moe_time_next_gemm applies to one GEMM call only: every
// GEMM entry point disarms it on return, whether or not it launched.
struct DisarmTiming {
  ~DisarmTiming() { moe::set_gemm_timing(nullptr, nullptr); }
};

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

moe_status moe_init(void) {
  clear_err();
  moe_status st = check_device("moe_init");
  if (st != MOE_OK) return st;
  // the device address of moe_route_noalloc's scratch, once per device
  void* p = nullptr;
  const hipError_t e = moe::route_scratch(&p);
  if (e != hipSuccess)
    return fail(MOE_E_HIP, "moe_init: grouping scratch lookup failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_time_next_gemm(void* start, void* stop) {
  clear_err();
  if ((start == nullptr) != (stop == nullptr))
    return fail(MOE_E_INVALID, "moe_time_next_gemm: start and stop must both be set or both NULL");
  moe::set_gemm_timing(static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
  return MOE_OK;
}

size_t moe_probe_out_values(void) { return (size_t)moe::kProbeBlocks * moe::kProbeThreads; }

double moe_probe_mfma_flops(int iters) {
  if (iters < 1) return 0.0;
  const double waves = (double)moe::kProbeBlocks * moe::kProbeThreads / 64.0;
  return waves * (double)iters * moe::kProbeMfmaChains * 32.0 * 32.0 * 16.0 * 2.0;
}

moe_status moe_probe_hbm_read(const void* buf, size_t bytes, uint32_t* out, moe_stream_t stream) {
  const char* fn = "moe_probe_hbm_read";
  DisarmTiming disarm;
  clear_err();
  REQUIRE_PTR(fn, buf);
  REQUIRE_PTR(fn, out);
  if (bytes < 16 || bytes % 16)
    return fail(MOE_E_INVALID, "%s: bytes=%zu must be a positive multiple of 16", fn, bytes);
  moe_status st = check_device(fn);
  if (st != MOE_OK) return st;
  return hip_status(fn, moe::launch_probe_read(buf, bytes, out, static_cast<hipStream_t>(stream)));
}

moe_status moe_probe_mfma_bf16(const uint16_t* ops, size_t n_ops, int iters, float* out,
                               moe_stream_t stream) {
  const char* fn = "moe_probe_mfma_bf16";
  DisarmTiming disarm;
  clear_err();
  REQUIRE_PTR(fn, ops);
  REQUIRE_PTR(fn, out);
  if (n_ops < 1 || n_ops > (1u << 26))
    return fail(MOE_E_INVALID, "%s: n_ops=%zu must be in [1, 2^26]", fn, n_ops);
  if (iters < 1 || iters > (1 << 20))
    return fail(MOE_E_INVALID, "%s: iters=%d must be in [1, 2^20]", fn, iters);
  moe_status st = check_device(fn);
  if (st != MOE_OK) return st;
  return hip_status(fn, moe::launch_probe_mfma(ops, (uint32_t)n_ops, iters, out,
                                               static_cast<hipStream_t>(stream)));
}

size_t moe_packed_weight_bytes(int E, int R, int K, moe_pack_kind kind) {
  if (E < 1 || R < 1 || K < 1 || K % 8 || (kind != MOE_PACK_PLAIN && kind != MOE_PACK_GATEUP))
    return 0;
  if (kind == MOE_PACK_GATEUP && R % 2) return 0;
  return (size_t)E * moe::packed_expert_bytes(R, K, kind == MOE_PACK_GATEUP);
}

moe_status moe_pack_weights(const uint16_t* w, int E, int R, int K, moe_pack_kind kind,
                            uint16_t* packed, moe_weights* desc, moe_stream_t stream) {
  const char* fn = "moe_pack_weights";
  clear_err();
  REQUIRE_NONNULL(fn, desc);
  if (kind != MOE_PACK_PLAIN && kind != MOE_PACK_GATEUP)
    return fail(MOE_E_INVALID, "%s: kind=%d is not MOE_PACK_PLAIN or MOE_PACK_GATEUP", fn,
                (int)kind);
  if (E < 1 || E > kMaxE) return fail(MOE_E_SHAPE, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (R < 1 || (kind == MOE_PACK_GATEUP && R % 2))
    return fail(MOE_E_SHAPE, "%s: R=%d must be positive (and even for MOE_PACK_GATEUP)", fn, R);
  if (K < 1 || K % 8) return fail(MOE_E_SHAPE, "%s: K=%d must be a positive multiple of 8", fn, K);
  if (!fits_packed(R, K, kind == MOE_PACK_GATEUP) || !fits_buf((long long)R * K))
    return fail(MOE_E_SHAPE, "%s: one expert's matrix [%d, %d] is too large", fn, R, K);
  REQUIRE_PTR(fn, w);
  REQUIRE_PTR(fn, packed);
  moe_status st = check_device(fn);
  if (st != MOE_OK) return st;
  st = hip_status(fn, moe::launch_pack(w, E, R, K, kind == MOE_PACK_GATEUP ? 1 : 0, packed,
                                       static_cast<hipStream_t>(stream)));
  if (st != MOE_OK) return st;
  moe_weights d{};
  d.layout = MOE_WEIGHTS_PACKED_V1;
  d.kind = (int32_t)kind;
  d.E = E;
  d.R = R;
  d.K = K;
  d.data = packed;
  d.expert_bytes = moe::packed_expert_bytes(R, K, kind == MOE_PACK_GATEUP);
  *desc = d;
  return MOE_OK;
}

moe_status moe_weights_slice(const moe_weights* w, int e0, int e1, moe_weights* out) {
  const char* fn = "moe_weights_slice";
  clear_err();
  REQUIRE_NONNULL(fn, w);
  REQUIRE_NONNULL(fn, out);
  if (w->layout != MOE_WEIGHTS_PACKED_V1)
    return fail(MOE_E_INVALID, "%s: w is not a packed weight descriptor (layout tag 0x%08x)", fn,
                w->layout);
  if (e0 < 0 || e1 <= e0 || e1 > w->E)
    return fail(MOE_E_SHAPE, "%s: expert range [%d, %d) outside [0, %d)", fn, e0, e1, w->E);
  moe_weights d = *w;
  d.E = e1 - e0;
  d.data = static_cast<const unsigned char*>(w->data) + (size_t)e0 * w->expert_bytes;
  *out = d;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Keep-quant path: Q8_K / Q8_0 activation buffers and the grouped GEMMs
// over Q4_K, Q5_K, Q6_K and Q8_0 weight blocks.
// ---------------------------------------------------------------------------
namespace {

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Q8KView {
  size_t qs, d, bs, total;  // byte offsets of the sections and the total size
};

Q8KView q8k_view(int R, int K) {
  Q8KView v;
  v.qs = 0;
  v.d = align256((size_t)R * K);
  v.bs = align256(v.d + (size_t)R * (K / 256) * 4);
  v.total = align256(v.bs + (size_t)R * (K / 16) * 4);
  return v;
}

bool q8k_shape_ok(int R, int K) {
  return R >= 0 && K >= 256 && K % 256 == 0 && (long long)R * K < (1LL << 31);
}

struct Q80View {
  size_t qs, d, total;
};

Q80View q8_0_view(int R, int K) {
  Q80View v;
  v.qs = 0;
  v.d = align256((size_t)R * K);
  v.total = align256(v.d + (size_t)R * (K / 32) * 2);
  return v;
}

bool q8_0_shape_ok(int R, int K) {
  return R >= 0 && K >= 32 && K % 32 == 0 && (long long)R * K < (1LL << 31);
}

// bytes of one weight row of Kd values
long long kq_row_bytes(moe_qtype wt, int Kd) {
  switch (wt) {
    case MOE_Q4_K: return (long long)(Kd / 256) * 144;
    case MOE_Q5_K: return (long long)(Kd / 256) * 176;
    case MOE_Q6_K: return (long long)(Kd / 256) * 210;
    case MOE_Q8_0: return (long long)(Kd / 32) * 34;
  }
  return 0;
}

// Section pointers of an activation buffer of the format that pairs with wt.
struct ActSections {
  const int8_t* qs;
  const void* d;
  const int32_t* bs;
};

ActSections act_sections(const void* buf, moe_qtype wt, int R, int K) {
  const unsigned char* b = static_cast<const unsigned char*>(buf);
  if (wt == MOE_Q8_0) {
    const Q80View v = q8_0_view(R, K);
    return {reinterpret_cast<const int8_t*>(b + v.qs), b + v.d, nullptr};
  }
  const Q8KView v = q8k_view(R, K);
  return {reinterpret_cast<const int8_t*>(b + v.qs), b + v.d,
          reinterpret_cast<const int32_t*>(b + v.bs)};
}

}  // namespace

size_t moe_q8k_bytes(int R, int K) {
  if (!q8k_shape_ok(R, K) || R == 0) return 0;
  return q8k_view(R, K).total;
}

moe_status moe_quantize_q8k(const uint16_t* x, int R, int K, void* xq, moe_stream_t stream) {
  const char* fn = "moe_quantize_q8k";
  clear_err();
  if (!q8k_shape_ok(R, K))
    return fail(MOE_E_SHAPE, "%s: K=%d must be a positive multiple of 256 and R*K below 2^31 "
                "(R=%d)", fn, K, R);
  if (R == 0) return MOE_OK;
  REQUIRE_PTR(fn, x);
  REQUIRE_PTR(fn, xq);
  moe_status st = check_device(fn);
  if (st != MOE_OK) return st;
  const Q8KView v = q8k_view(R, K);
  unsigned char* b = static_cast<unsigned char*>(xq);
  return hip_status(fn, moe::launch_quantize_q8k(x, R, K, reinterpret_cast<int8_t*>(b + v.qs),
                                                 reinterpret_cast<float*>(b + v.d),
                                                 reinterpret_cast<int32_t*>(b + v.bs),
                                                 static_cast<hipStream_t>(stream)));
}

size_t moe_q8_0_bytes(int R, int K) {
  if (!q8_0_shape_ok(R, K) || R == 0) return 0;
  return q8_0_view(R, K).total;
}

moe_status moe_quantize_q8_0(const uint16_t* x, int R, int K, void* xq, moe_stream_t stream) {
  const char* fn = "moe_quantize_q8_0";
  clear_err();
  if (!q8_0_shape_ok(R, K))
    return fail(MOE_E_SHAPE, "%s: K=%d must be a positive multiple of 32 and R*K below 2^31 "
                "(R=%d)", fn, K, R);
  if (R == 0) return MOE_OK;
  REQUIRE_PTR(fn, x);
  REQUIRE_PTR(fn, xq);
  moe_status st = check_device(fn);
  if (st != MOE_OK) return st;
  const Q80View v = q8_0_view(R, K);
  unsigned char* b = static_cast<unsigned char*>(xq);
  return hip_status(fn, moe::launch_quantize_q8_0(x, R, K, reinterpret_cast<int8_t*>(b + v.qs),
                                                  reinterpret_cast<uint16_t*>(b + v.d),
                                                  static_cast<hipStream_t>(stream)));
}

static moe_status kq_common(const char* fn, moe_qtype wt, int E, int R, int Kd) {
  if (wt != MOE_Q4_K && wt != MOE_Q5_K && wt != MOE_Q6_K && wt != MOE_Q8_0)
    return fail(MOE_E_DTYPE,
                "%s: weight type %d unsupported (MOE_Q8_0, MOE_Q4_K, MOE_Q5_K or MOE_Q6_K)", fn,
                (int)wt);
  if (E < 1 || E > kMaxE) return fail(MOE_E_SHAPE, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (Kd < 256 || Kd % 256)
    return fail(MOE_E_SHAPE, "%s: the reduced dimension %d must be a positive multiple of 256", fn,
                Kd);
  if ((long long)R * kq_row_bytes(wt, Kd) >= (1LL << 31))
    return fail(MOE_E_SHAPE, "%s: one expert's weight blocks exceed 2^31 bytes", fn);
  return MOE_OK;
}

moe_status moe_grouped_qgemm_gateup_silu(const void* xq, int T, int H, const void* w_gu,
                                         moe_qtype wt, int E, int I, const int32_t* sorted_pairs,
                                         const int32_t* expert_offsets, int K, uint16_t* act,
                                         moe_stream_t stream) {
  const char* fn = "moe_grouped_qgemm_gateup_silu";
  DisarmTiming disarm;
  clear_err();
  if (T < 0) return fail(MOE_E_SHAPE, "%s: T=%d is negative", fn, T);
  moe_status st = kq_common(fn, wt, E, 2 * I, H);
  if (st != MOE_OK) return st;
  if (I <= 0 || I % 8) return fail(MOE_E_SHAPE, "%s: I=%d must be a positive multiple of 8", fn, I);
  if (K < 1 || K > E || K > kMaxK)
    return fail(MOE_E_SHAPE, "%s: K=%d outside [1, min(E=%d, %d)]", fn, K, E, kMaxK);
  if ((sorted_pairs == nullptr) != (expert_offsets == nullptr))
    return fail(MOE_E_INVALID, "%s: sorted_pairs and expert_offsets must both be set or both NULL",
                fn);
  if (sorted_pairs == nullptr && (E != 1 || K != 1))
    return fail(MOE_E_INVALID, "%s: identity rows (NULL sorted_pairs) need E=1 and K=1, got E=%d K=%d",
                fn, E, K);
  if (!q8k_shape_ok(T, H) || !fits_i32((long long)T * K * I))
    return fail(MOE_E_SHAPE, "%s: T*H or T*K*I exceeds 2^31", fn);
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(fn, xq);
  REQUIRE_PTR(fn, w_gu);
  REQUIRE_PTR(fn, act);
  st = check_device(fn);
  if (st != MOE_OK) return st;
  const ActSections a = act_sections(xq, wt, T, H);
  return hip_status(fn, moe::launch_kq_gateup_silu(a.qs, a.d, a.bs, T, H,
                                                   static_cast<const uint8_t*>(w_gu), (int)wt, E, I,
                                                   sorted_pairs, expert_offsets, K, act,
                                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_qgemm_down(const void* actq, int P, int I, const void* w_d, moe_qtype wt,
                                  int E, int H, const int32_t* sorted_pairs,
                                  const int32_t* expert_offsets, const float* pair_w,
                                  uint16_t* expert_out, moe_stream_t stream) {
  const char* fn = "moe_grouped_qgemm_down";
  DisarmTiming disarm;
  clear_err();
  if (P < 0) return fail(MOE_E_SHAPE, "%s: P=%d is negative", fn, P);
  moe_status st = kq_common(fn, wt, E, H, I);
  if (st != MOE_OK) return st;
  if (H <= 0 || H % 8) return fail(MOE_E_SHAPE, "%s: H=%d must be a positive multiple of 8", fn, H);
  if ((sorted_pairs == nullptr) != (expert_offsets == nullptr))
    return fail(MOE_E_INVALID, "%s: sorted_pairs and expert_offsets must both be set or both NULL",
                fn);
  if (sorted_pairs == nullptr && E != 1)
    return fail(MOE_E_INVALID, "%s: identity rows (NULL sorted_pairs) need E=1, got E=%d", fn, E);
  if (!q8k_shape_ok(P, I) || !fits_i32((long long)P * H))
    return fail(MOE_E_SHAPE, "%s: P*I or P*H exceeds 2^31", fn);
  if (P == 0) return MOE_OK;
  REQUIRE_PTR(fn, actq);
  REQUIRE_PTR(fn, w_d);
  REQUIRE_PTR(fn, expert_out);
  st = check_device(fn);
  if (st != MOE_OK) return st;
  const ActSections a = act_sections(actq, wt, P, I);
  return hip_status(fn, moe::launch_kq_down(a.qs, a.d, a.bs, P, I, static_cast<const uint8_t*>(w_d),
                                            (int)wt, E, H, sorted_pairs, expert_offsets, pair_w,
                                            expert_out, static_cast<hipStream_t>(stream)));
}

moe_status moe_router_logits(const uint16_t* x, int T, int H, const uint16_t* w, int N,
                             const float* bias, float* out, moe_stream_t stream) {
  const char* fn = "moe_router_logits";
  DisarmTiming disarm;
  clear_err();
  if (T < 0) return fail(MOE_E_SHAPE, "%s: T=%d is negative", fn, T);
  if (H <= 0 || H % 8) return fail(MOE_E_SHAPE, "%s: H=%d must be a positive multiple of 8", fn, H);
  if (N < 1) return fail(MOE_E_SHAPE, "%s: N=%d must be >= 1", fn, N);
  if (!fits_buf((long long)T * H) || !fits_i32((long long)T * N) || !fits_buf((long long)N * H))
    return fail(MOE_E_SHAPE, "%s: T*H or N*H exceeds 2^30 elements, or T*N 2^31", fn);
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(fn, x);
  REQUIRE_PTR(fn, w);
  REQUIRE_NONNULL(fn, out);
  moe_status st = check_device(fn);
  if (st != MOE_OK) return st;
  return hip_status(fn, moe::launch_logits(x, T, H, w, N, bias, out,
                                           static_cast<hipStream_t>(stream)));
}

size_t moe_route_workspace_bytes(int T, int E, int K) {
  if (T <= 0 || E < 1 || K < 1) return 0;
  return moe::route_workspace_bytes(T, E, K);
}

moe_status moe_route(const float* logits, int T, int E, int K, int32_t* topk_ids, float* topk_w,
                     int32_t* expert_offsets, int32_t* sorted_pairs, void* ws, size_t ws_bytes,
                     moe_stream_t stream) {
  const char* fn = "moe_route";
  clear_err();
  if (T < 0) return fail(MOE_E_SHAPE, "%s: T=%d is negative", fn, T);
  if (E < 1 || E > kMaxE) return fail(MOE_E_SHAPE, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (K < 1 || K > E || K > kMaxK)
    return fail(MOE_E_SHAPE, "%s: K=%d outside [1, min(E=%d, %d)]", fn, K, E, kMaxK);
  if (!fits_i32((long long)T * E) || !fits_i32((long long)T * K))
    return fail(MOE_E_SHAPE, "%s: T*E or T*K exceeds 2^31", fn);
  if (ws_bytes < moe_route_workspace_bytes(T, E, K))
    return fail(MOE_E_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, ws_bytes,
                moe_route_workspace_bytes(T, E, K));
  REQUIRE_NONNULL(fn, expert_offsets);
  if (T == 0) return MOE_OK;  // nothing routed; no output is written
  if (moe_route_workspace_bytes(T, E, K) > 0 && (ws == nullptr || (uintptr_t)ws % 4 != 0))
    return fail(MOE_E_WORKSPACE, "%s: ws is NULL or not 4-byte aligned (%zu bytes needed)", fn,
                moe_route_workspace_bytes(T, E, K));
  REQUIRE_NONNULL(fn, logits);
  REQUIRE_NONNULL(fn, topk_ids);
  REQUIRE_NONNULL(fn, topk_w);
  REQUIRE_NONNULL(fn, sorted_pairs);
  moe_status st = check_device(fn);
  if (st != MOE_OK) return st;
  return hip_status(fn, moe::launch_route(logits, T, E, K, topk_ids, topk_w, expert_offsets,
                                          sorted_pairs, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_route_noalloc(const float* logits, int T, int E, int K, int32_t* topk_ids,
                             float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                             moe_stream_t stream) {
  const char* fn = "moe_route_noalloc";
  clear_err();
  if (T < 0) return fail(MOE_E_SHAPE, "%s: T=%d is negative", fn, T);
  if (E < 1 || E > kMaxE) return fail(MOE_E_SHAPE, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (K < 1 || K > E || K > kMaxK)
    return fail(MOE_E_SHAPE, "%s: K=%d outside [1, min(E=%d, %d)]", fn, K, E, kMaxK);
  if (!fits_i32((long long)T * E) || !fits_i32((long long)T * K))
    return fail(MOE_E_SHAPE, "%s: T*E or T*K exceeds 2^31", fn);
  const size_t need = moe_route_workspace_bytes(T, E, K);
  if (need > moe::kRouteScratchBytes)
    return fail(MOE_E_WORKSPACE,
                "%s: T*K=%lld pairs over E=%d experts need %zu bytes of grouping scratch; the "
                "library holds %zu (use moe_route with a caller workspace)",
                fn, (long long)T * K, E, need, moe::kRouteScratchBytes);
  REQUIRE_NONNULL(fn, expert_offsets);
  if (T == 0) return MOE_OK;  // nothing routed; no output is written
  REQUIRE_NONNULL(fn, logits);
  REQUIRE_NONNULL(fn, topk_ids);
  REQUIRE_NONNULL(fn, topk_w);
  REQUIRE_NONNULL(fn, sorted_pairs);
  moe_status st = check_device(fn);
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  const hipError_t e = moe::route_scratch(&ws);
  if (e != hipSuccess)
    return fail(MOE_E_HIP, "%s: grouping scratch lookup failed: %s", fn, hipGetErrorString(e));
  return hip_status(fn, moe::launch_route(logits, T, E, K, topk_ids, topk_w, expert_offsets,
                                          sorted_pairs, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_route_scored(const float* logits, int T, int E, int K, moe_score score,
                            const float* selection_bias, int n_group, int topk_group,
                            moe_group_score group_score, int renormalize, int32_t* topk_ids,
                            float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                            void* ws, size_t ws_bytes, moe_stream_t stream) {
  const char* fn = "moe_route_scored";
  clear_err();
  if (T < 0) return fail(MOE_E_SHAPE, "%s: T=%d is negative", fn, T);
  if (E < 1 || E > kMaxE) return fail(MOE_E_SHAPE, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (K < 1 || K > E || K > kMaxK)
    return fail(MOE_E_SHAPE, "%s: K=%d outside [1, min(E=%d, %d)]", fn, K, E, kMaxK);
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)
    return fail(MOE_E_INVALID, "%s: score=%d is not MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID", fn,
                (int)score);
  if (group_score != MOE_GROUP_MAX && group_score != MOE_GROUP_TOP2_SUM)
    return fail(MOE_E_INVALID, "%s: group_score=%d is not MOE_GROUP_MAX or MOE_GROUP_TOP2_SUM",
                fn, (int)group_score);
  if (renormalize != 0 && renormalize != 1)
    return fail(MOE_E_INVALID, "%s: renormalize=%d must be 0 or 1", fn, renormalize);
  if (n_group < 1 || n_group > 64 || E % n_group != 0)
    return fail(MOE_E_SHAPE, "%s: n_group=%d must divide E=%d and lie in [1, 64]", fn, n_group,
                E);
  if (topk_group < 1 || topk_group > n_group)
    return fail(MOE_E_SHAPE, "%s: topk_group=%d outside [1, n_group=%d]", fn, topk_group,
                n_group);
  if ((long long)topk_group * (E / n_group) < K)
    return fail(MOE_E_SHAPE, "%s: %d groups of %d experts hold fewer than K=%d experts", fn,
                topk_group, E / n_group, K);
  if (!fits_i32((long long)T * E) || !fits_i32((long long)T * K))
    return fail(MOE_E_SHAPE, "%s: T*E or T*K exceeds 2^31", fn);
  if (ws_bytes < moe_route_workspace_bytes(T, E, K))
    return fail(MOE_E_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, ws_bytes,
                moe_route_workspace_bytes(T, E, K));
  REQUIRE_NONNULL(fn, expert_offsets);
  if (T == 0) return MOE_OK;  // nothing routed; no output is written
  if (moe_route_workspace_bytes(T, E, K) > 0 && (ws == nullptr || (uintptr_t)ws % 4 != 0))
    return fail(MOE_E_WORKSPACE, "%s: ws is NULL or not 4-byte aligned (%zu bytes needed)", fn,
                moe_route_workspace_bytes(T, E, K));
  REQUIRE_NONNULL(fn, logits);
  REQUIRE_NONNULL(fn, topk_ids);
  REQUIRE_NONNULL(fn, topk_w);
  REQUIRE_NONNULL(fn, sorted_pairs);
  moe_status st = check_device(fn);
  if (st != MOE_OK) return st;
  return hip_status(
      fn, moe::launch_route_scored(logits, T, E, K, score == MOE_SCORE_SIGMOID ? 1 : 0,
                                   selection_bias, n_group, topk_group,
                                   group_score == MOE_GROUP_TOP2_SUM ? 1 : 0, renormalize,
                                   topk_ids, topk_w, expert_offsets, sorted_pairs, ws,
                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_gemm_gateup_silu(const uint16_t* x, int T, int H, const moe_weights* w_gu,
                                        int E, int I, const int32_t* sorted_pairs,
                                        const int32_t* expert_offsets, int K, uint16_t* act,
                                        moe_stream_t stream) {
  const char* fn = "moe_grouped_gemm_gateup_silu";
  DisarmTiming disarm;
  clear_err();
  if (T < 0) return fail(MOE_E_SHAPE, "%s: T=%d is negative", fn, T);
  if (H <= 0 || H % 8) return fail(MOE_E_SHAPE, "%s: H=%d must be a positive multiple of 8", fn, H);
  if (I <= 0 || I % 8) return fail(MOE_E_SHAPE, "%s: I=%d must be a positive multiple of 8", fn, I);
  if (E < 1 || E > kMaxE) return fail(MOE_E_SHAPE, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (K < 1 || K > E || K > kMaxK)
    return fail(MOE_E_SHAPE, "%s: K=%d outside [1, min(E=%d, %d)]", fn, K, E, kMaxK);
  if ((sorted_pairs == nullptr) != (expert_offsets == nullptr))
    return fail(MOE_E_INVALID, "%s: sorted_pairs and expert_offsets must both be set or both NULL",
                fn);
  if (sorted_pairs == nullptr && (E != 1 || K != 1))
    return fail(MOE_E_INVALID, "%s: identity rows (NULL sorted_pairs) need E=1 and K=1, got E=%d K=%d",
                fn, E, K);
  if (!fits_i32((long long)T * K) || !fits_buf((long long)T * H) ||
      !fits_i32((long long)T * K * I) || !fits_packed(2 * I, H, true))
    return fail(MOE_E_SHAPE, "%s: x exceeds 2^30 elements, one expert's packed w_gu 2^31 bytes, or T*K*I 2^31",
                fn);
  if (T == 0) return MOE_OK;
  moe_status st = check_weights(fn, "w_gu", w_gu, MOE_PACK_GATEUP, E, 2 * I, H);
  if (st != MOE_OK) return st;
  REQUIRE_PTR(fn, x);
  REQUIRE_PTR(fn, act);
  st = check_device(fn);
  if (st != MOE_OK) return st;
  return hip_status(fn, moe::launch_gateup_silu(x, T, H, static_cast<const uint16_t*>(w_gu->data),
                                                E, I, sorted_pairs, expert_offsets, K, act,
                                                static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_gemm_down(const uint16_t* act, int P, int I, const moe_weights* w_d,
                                 int E, int H, const int32_t* sorted_pairs,
                                 const int32_t* expert_offsets, const float* pair_w,
                                 uint16_t* expert_out, moe_stream_t stream) {
  const char* fn = "moe_grouped_gemm_down";
  DisarmTiming disarm;
  clear_err();
  if (P < 0) return fail(MOE_E_SHAPE, "%s: P=%d is negative", fn, P);
  if (H <= 0 || H % 8) return fail(MOE_E_SHAPE, "%s: H=%d must be a positive multiple of 8", fn, H);
  if (I <= 0 || I % 8) return fail(MOE_E_SHAPE, "%s: I=%d must be a positive multiple of 8", fn, I);
  if (E < 1 || E > kMaxE) return fail(MOE_E_SHAPE, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if ((sorted_pairs == nullptr) != (expert_offsets == nullptr))
    return fail(MOE_E_INVALID, "%s: sorted_pairs and expert_offsets must both be set or both NULL",
                fn);
  if (sorted_pairs == nullptr && E != 1)
    return fail(MOE_E_INVALID, "%s: identity rows (NULL sorted_pairs) need E=1, got E=%d", fn, E);
  if (!fits_buf((long long)P * I) || !fits_i32((long long)P * H) || !fits_packed(H, I, false))
    return fail(MOE_E_SHAPE,
                "%s: act exceeds 2^30 elements, one expert's packed w_d 2^31 bytes, or P*H 2^31", fn);
  if (P == 0) return MOE_OK;
  moe_status st = check_weights(fn, "w_d", w_d, MOE_PACK_PLAIN, E, H, I);
  if (st != MOE_OK) return st;
  REQUIRE_PTR(fn, act);
  REQUIRE_PTR(fn, expert_out);
  st = check_device(fn);
  if (st != MOE_OK) return st;
  return hip_status(fn, moe::launch_down(act, P, I, static_cast<const uint16_t*>(w_d->data), E, H,
                                         sorted_pairs, expert_offsets, pair_w, expert_out,
                                         static_cast<hipStream_t>(stream)));
}

size_t moe_fused_expert_ffn_workspace_bytes(int T, int E, int K, int grouped) {
  if (T <= 0 || E < 1 || K < 1 || !fits_i32((long long)T * K)) return 0;
  return (size_t)moe::fused_ffn_workspace_ints(T * K, E, grouped != 0) * 4;
}

moe_status moe_fused_expert_ffn(const uint16_t* x, int T, int H, const moe_weights* w_gu,
                                const moe_weights* w_d, int E, int I, const int32_t* sorted_pairs,
                                const int32_t* expert_offsets, int K, const float* pair_w,
                                uint16_t* act, uint16_t* expert_out, void* ws, size_t ws_bytes,
                                moe_stream_t stream) {
  const char* fn = "moe_fused_expert_ffn";
  DisarmTiming disarm;
  clear_err();
  if (T < 0) return fail(MOE_E_SHAPE, "%s: T=%d is negative", fn, T);
  if (H <= 0 || H % 8) return fail(MOE_E_SHAPE, "%s: H=%d must be a positive multiple of 8", fn, H);
  if (I <= 0 || I % 8) return fail(MOE_E_SHAPE, "%s: I=%d must be a positive multiple of 8", fn, I);
  if (E < 1 || E > kMaxE) return fail(MOE_E_SHAPE, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  if (K < 1 || K > E || K > kMaxK)
    return fail(MOE_E_SHAPE, "%s: K=%d outside [1, min(E=%d, %d)]", fn, K, E, kMaxK);
  if ((sorted_pairs == nullptr) != (expert_offsets == nullptr))
    return fail(MOE_E_INVALID, "%s: sorted_pairs and expert_offsets must both be set or both NULL",
                fn);
  if (sorted_pairs == nullptr && (E != 1 || K != 1))
    return fail(MOE_E_INVALID, "%s: identity rows (NULL sorted_pairs) need E=1 and K=1, got E=%d K=%d",
                fn, E, K);
  if (!fits_i32((long long)T * K) || !fits_buf((long long)T * H) ||
      !fits_buf((long long)T * K * I) || !fits_i32((long long)T * K * H) ||
      !fits_packed(2 * I, H, true) || !fits_packed(H, I, false))
    return fail(MOE_E_SHAPE, "%s: x or act exceeds 2^30 elements, T*K*H 2^31, or one expert's packed "
                "weights 2^31 bytes", fn);
  const int grouped = sorted_pairs != nullptr;
  const size_t need = moe_fused_expert_ffn_workspace_bytes(T, E, K, grouped);
  if (T > 0 && ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, ws_bytes, need);
  if (T == 0) return MOE_OK;
  moe_status st = check_weights(fn, "w_gu", w_gu, MOE_PACK_GATEUP, E, 2 * I, H);
  if (st != MOE_OK) return st;
  st = check_weights(fn, "w_d", w_d, MOE_PACK_PLAIN, E, H, I);
  if (st != MOE_OK) return st;
  if (ws == nullptr || (uintptr_t)ws % 4 != 0)
    return fail(MOE_E_WORKSPACE, "%s: ws is NULL or not 4-byte aligned (%zu bytes needed)", fn, need);
  REQUIRE_PTR(fn, x);
  REQUIRE_PTR(fn, act);
  REQUIRE_PTR(fn, expert_out);
  st = check_device(fn);
  if (st != MOE_OK) return st;
  return hip_status(fn, moe::launch_fused_ffn(x, T, H, static_cast<const uint16_t*>(w_gu->data),
                                              static_cast<const uint16_t*>(w_d->data), E, I,
                                              sorted_pairs,
                                              expert_offsets, K, pair_w, act, expert_out,
                                              static_cast<int*>(ws),
                                              static_cast<hipStream_t>(stream)));
}

moe_status moe_combine_gate(const void* expert_out, moe_dtype eo_dt, int T, int K, int H,
                            const float* topk_w, float routed_scale, const void* shared,
                            moe_dtype sh_dt, const float* gate_logit, void* out,
                            moe_dtype out_dt, moe_stream_t stream) {
  const char* fn = "moe_combine_gate";
  clear_err();
  DisarmTiming disarm;
  moe_status st = check_dtype(fn, "expert_out", eo_dt);
  if (st != MOE_OK) return st;
  if (shared != nullptr) {
    st = check_dtype(fn, "shared", sh_dt);
    if (st != MOE_OK) return st;
  }
  st = check_dtype(fn, "out", out_dt);
  if (st != MOE_OK) return st;
  if (T < 0) return fail(MOE_E_SHAPE, "%s: T=%d is negative", fn, T);
  if (K < 1 || K > kMaxK) return fail(MOE_E_SHAPE, "%s: K=%d outside [1, %d]", fn, K, kMaxK);
  if (H <= 0 || H % 8) return fail(MOE_E_SHAPE, "%s: H=%d must be a positive multiple of 8", fn, H);
  if (!fits_i32((long long)T * K * H))
    return fail(MOE_E_SHAPE, "%s: T*K*H exceeds 2^31 elements", fn);
  if (!std::isfinite(routed_scale))
    return fail(MOE_E_INVALID, "%s: routed_scale is not finite", fn);
  if (gate_logit != nullptr && shared == nullptr)
    return fail(MOE_E_INVALID, "%s: gate_logit given without a shared term", fn);
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(fn, expert_out);
  REQUIRE_PTR(fn, out);
  if (shared != nullptr && !aligned16(shared))
    return fail(MOE_E_INVALID, "%s: shared is not 16-byte aligned", fn);
  st = check_device(fn);
  if (st != MOE_OK) return st;
  return hip_status(fn, moe::launch_combine(expert_out, eo_dt == MOE_BF16, T, K, H, topk_w,
                                            routed_scale, shared, sh_dt == MOE_BF16, gate_logit,
                                            out, out_dt == MOE_BF16,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
