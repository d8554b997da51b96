// C ABI of the shallow-state engine (declared in include/seed.h).
//
// Every entry point validates its arguments on the host first and returns a
// status without touching the HIP runtime when they are wrong; only valid
// calls reach the launchers.  The library keeps no state besides a
// thread-local error message.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/seed.h"
#include "seed_launch.h"

namespace {

thread_local char g_err[512] = "";

seed_status fail(seed_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

seed_status ok() {
  g_err[0] = '\0';
  return SEED_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define SEED_PTR(p)                                                                     \
  do {                                                                                  \
    if ((p) == nullptr) return fail(SEED_E_ARG, "%s: %s is NULL", fn, #p);              \
    if (!aligned16(p)) return fail(SEED_E_ARG, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

bool supported_dims(int d_k, int d_v) {
  return (d_k == 128 && d_v == 128) || (d_k == 128 && d_v == 64) || (d_k == 64 && d_v == 64);
}

seed_status check_units(const char* fn, int batch, int heads, int d_k, int d_v) {
  if (batch <= 0 || heads <= 0 || d_k <= 0 || d_v <= 0)
    return fail(SEED_E_SHAPE, "%s: batch, heads, d_k, d_v must be positive (got %d, %d, %d, %d)",
                fn, batch, heads, d_k, d_v);
  if ((long long)batch * heads > 0x7fffffffLL)
    return fail(SEED_E_SHAPE, "%s: batch * heads = %lld exceeds the grid limit", fn,
                (long long)batch * heads);
  if (!supported_dims(d_k, d_v))
    return fail(SEED_E_UNSUPPORTED,
                "%s: head shape d_k=%d d_v=%d not supported (use 128x128, 128x64 or 64x64)", fn,
                d_k, d_v);
  return SEED_OK;
}

seed_status check_step_inputs(const char* fn, int rule, const void* q, const void* k,
                              const void* v, int in_dtype, const float* g, const float* beta,
                              float* o) {
  if (rule != SEED_RULE_GDN && rule != SEED_RULE_KDA && rule != SEED_RULE_MAMBA2)
    return fail(SEED_E_ARG, "%s: unknown rule %d", fn, rule);
  if (in_dtype != SEED_F32 && in_dtype != SEED_BF16)
    return fail(SEED_E_ARG, "%s: unknown input dtype %d", fn, in_dtype);
  SEED_PTR(q);
  SEED_PTR(k);
  SEED_PTR(v);
  SEED_PTR(g);
  SEED_PTR(o);
  if (rule == SEED_RULE_MAMBA2) {
    if (beta != nullptr) return fail(SEED_E_ARG, "%s: beta must be NULL for Mamba-2", fn);
  } else {
    SEED_PTR(beta);
  }
  return SEED_OK;
}

seed_status device_status(const char* fn, hipError_t e) {
  if (e != hipSuccess)
    return fail(SEED_E_DEVICE, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace {

seed_status decode_step(const char* fn, int rule, int batch, int heads, int d_k, int d_v, int cap,
                        int r, float* a, float* U, float* V, float* gam, bool lazy,
                        const float* vbar, const void* q, const void* k, const void* v,
                        int in_dtype, const float* g, const float* beta, float* o, void* stream) {
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  if (cap <= 0 || r < 0 || r > cap)
    return fail(SEED_E_SHAPE, "%s: need 0 <= r <= cap, cap > 0 (got r=%d cap=%d)", fn, r, cap);
  if (cap > seed::kMaxCap)
    return fail(SEED_E_UNSUPPORTED, "%s: capacity %d above %d", fn, cap, seed::kMaxCap);
  if (r == cap)
    return fail(SEED_E_FULL, "%s: all %d columns are in use; compress first", fn, cap);
  st = check_step_inputs(fn, rule, q, k, v, in_dtype, g, beta, o);
  if (st != SEED_OK) return st;
  SEED_PTR(a);
  SEED_PTR(U);
  SEED_PTR(V);
  SEED_PTR(vbar);
  if (lazy) SEED_PTR(gam);
  return device_status(fn, seed::launch_step(rule, in_dtype == SEED_BF16, seed::kStoreF32, batch,
                                             heads, d_k, d_v, cap, r, 0, a, U, V, nullptr, nullptr,
                                             lazy ? gam : nullptr, vbar, q, k, v, g, beta, o,
                                             static_cast<hipStream_t>(stream)));
}

int store_fmt_of(int store_dtype) {
  return store_dtype == SEED_BF16 ? seed::kStoreBF16 : seed::kStoreF16;
}

// Shapes of the 16-bit form: R kept columns, a window of W fp32 columns,
// r columns held in all.
seed_status check_h16(const char* fn, int batch, int heads, int d_k, int d_v, int R, int W, int r,
                      int store_dtype) {
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  if (store_dtype != SEED_BF16 && store_dtype != SEED_F16)
    return fail(SEED_E_ARG, "%s: store dtype must be SEED_BF16 or SEED_F16 (got %d)", fn,
                store_dtype);
  if (R <= 0 || W <= 0 || r < R || r > R + W)
    return fail(SEED_E_SHAPE, "%s: need R > 0, W > 0 and R <= r <= R + W (got R=%d W=%d r=%d)", fn,
                R, W, r);
  if (R + W > seed::kMaxCap)
    return fail(SEED_E_UNSUPPORTED, "%s: capacity R + W = %d above %d", fn, R + W, seed::kMaxCap);
  if (R != 16 && R != 32)
    return fail(SEED_E_UNSUPPORTED, "%s: the 16-bit form is built for R = 16 or 32 (got %d)", fn,
                R);
  return SEED_OK;
}

seed_status compress(const char* fn, int rule, int batch, int heads, int d_k, int d_v, int cap,
                     int r, int R, float* U, float* V, float* gam, bool lazy, void* stream) {
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  if (lazy && rule != SEED_RULE_GDN && rule != SEED_RULE_KDA && rule != SEED_RULE_MAMBA2)
    return fail(SEED_E_ARG, "%s: unknown rule %d", fn, rule);
  if (cap <= 0 || R <= 0 || r < 0 || r > cap || R > cap)
    return fail(SEED_E_SHAPE, "%s: need 0 < R <= cap and 0 <= r <= cap (got R=%d r=%d cap=%d)",
                fn, R, r, cap);
  if (cap > seed::kMaxCap)
    return fail(SEED_E_UNSUPPORTED, "%s: capacity %d above %d", fn, cap, seed::kMaxCap);
  if (R > 32) return fail(SEED_E_UNSUPPORTED, "%s: rank %d above 32", fn, R);
  SEED_PTR(U);
  SEED_PTR(V);
  if (lazy) SEED_PTR(gam);
  if (r <= R) return ok();
  if (seed::compress_lds_bytes(r, R) > seed::kMaxLds)
    return fail(SEED_E_UNSUPPORTED, "%s: %d columns at rank %d need more LDS than a CU has", fn,
                r, R);
  seed::CompressArgs args{batch * heads, cap, r, R, U, V, nullptr, nullptr,
                          lazy ? gam : nullptr, rule == SEED_RULE_KDA, 0, 0u, 0u, 0u};
  return device_status(fn, seed::launch_compress(d_k, d_v, seed::kStoreF32, args,
                                                 static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

seed_status seed_decode_step(int rule, int batch, int heads, int d_k, int d_v, int cap, int r,
                             float* a, float* U, float* V, const float* vbar, const void* q,
                             const void* k, const void* v, int in_dtype, const float* g,
                             const float* beta, float* o, void* stream) {
  return decode_step("seed_decode_step", rule, batch, heads, d_k, d_v, cap, r, a, U, V, nullptr,
                     false, vbar, q, k, v, in_dtype, g, beta, o, stream);
}

seed_status seed_decode_step_lazy(int rule, int batch, int heads, int d_k, int d_v, int cap,
                                  int r, float* a, float* U, float* V, float* gam,
                                  const float* vbar, const void* q, const void* k, const void* v,
                                  int in_dtype, const float* g, const float* beta, float* o,
                                  void* stream) {
  return decode_step("seed_decode_step_lazy", rule, batch, heads, d_k, d_v, cap, r, a, U, V, gam,
                     true, vbar, q, k, v, in_dtype, g, beta, o, stream);
}

seed_status seed_compress(int batch, int heads, int d_k, int d_v, int cap, int r, int R,
                          float* U, float* V, void* stream) {
  return compress("seed_compress", SEED_RULE_GDN, batch, heads, d_k, d_v, cap, r, R, U, V,
                  nullptr, false, stream);
}

seed_status seed_compress_lazy(int rule, int batch, int heads, int d_k, int d_v, int cap, int r,
                               int R, float* U, float* V, float* gam, void* stream) {
  return compress("seed_compress_lazy", rule, batch, heads, d_k, d_v, cap, r, R, U, V, gam, true,
                  stream);
}

seed_status seed_decode_step_h16(int rule, int batch, int heads, int d_k, int d_v, int R, int W,
                                 int r, float* a, void* Uk, const void* Vk, float* Uw,
                                 float* Vw, float* gam, const float* vbar, const void* q,
                                 const void* k, const void* v, int in_dtype, int store_dtype,
                                 const float* g, const float* beta, float* o, void* stream) {
  const char* fn = "seed_decode_step_h16";
  seed_status st = check_h16(fn, batch, heads, d_k, d_v, R, W, r, store_dtype);
  if (st != SEED_OK) return st;
  if (r == R + W)
    return fail(SEED_E_FULL, "%s: all %d window columns are in use; compress first", fn, W);
  st = check_step_inputs(fn, rule, q, k, v, in_dtype, g, beta, o);
  if (st != SEED_OK) return st;
  SEED_PTR(a);
  SEED_PTR(Uk);
  SEED_PTR(Vk);
  SEED_PTR(Uw);
  SEED_PTR(Vw);
  SEED_PTR(gam);
  SEED_PTR(vbar);
  return device_status(
      fn, seed::launch_step(rule, in_dtype == SEED_BF16, store_fmt_of(store_dtype), batch, heads,
                            d_k, d_v, W, r, R, a, Uw, Vw, static_cast<uint16_t*>(Uk),
                            static_cast<const uint16_t*>(Vk), gam, vbar, q, k, v, g, beta, o,
                            static_cast<hipStream_t>(stream)));
}

seed_status seed_compress_h16(int rule, int batch, int heads, int d_k, int d_v, int R, int W,
                              int r, void* Uk, void* Vk, float* Uw, float* Vw, float* gam,
                              int store_dtype, int rounding, uint64_t seed, uint32_t epoch,
                              void* stream) {
  const char* fn = "seed_compress_h16";
  seed_status st = check_h16(fn, batch, heads, d_k, d_v, R, W, r, store_dtype);
  if (st != SEED_OK) return st;
  if (rule != SEED_RULE_GDN && rule != SEED_RULE_KDA && rule != SEED_RULE_MAMBA2)
    return fail(SEED_E_ARG, "%s: unknown rule %d", fn, rule);
  if (rounding != SEED_ROUND_NEAREST && rounding != SEED_ROUND_STOCHASTIC)
    return fail(SEED_E_ARG, "%s: unknown rounding %d", fn, rounding);
  SEED_PTR(Uk);
  SEED_PTR(Vk);
  SEED_PTR(Uw);
  SEED_PTR(Vw);
  SEED_PTR(gam);
  if (r <= R) return ok();
  if (seed::compress_lds_bytes(r, R) > seed::kMaxLds)
    return fail(SEED_E_UNSUPPORTED, "%s: %d columns at rank %d need more LDS than a CU has", fn,
                r, R);
  seed::CompressArgs args{batch * heads, W, r, R, Uw, Vw,
                          static_cast<uint16_t*>(Uk), static_cast<uint16_t*>(Vk), gam,
                          rule == SEED_RULE_KDA, rounding == SEED_ROUND_STOCHASTIC, epoch,
                          (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  return device_status(fn, seed::launch_compress(d_k, d_v, store_fmt_of(store_dtype), args,
                                                 static_cast<hipStream_t>(stream)));
}

seed_status seed_round_factors(int batch, int heads, int d_k, int d_v, int R, const float* U,
                               const float* V, void* Uk, void* Vk, int store_dtype, int rounding,
                               uint64_t seed, uint32_t epoch, void* stream) {
  const char* fn = "seed_round_factors";
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  if (store_dtype != SEED_BF16 && store_dtype != SEED_F16)
    return fail(SEED_E_ARG, "%s: store dtype must be SEED_BF16 or SEED_F16 (got %d)", fn,
                store_dtype);
  if (rounding != SEED_ROUND_NEAREST && rounding != SEED_ROUND_STOCHASTIC)
    return fail(SEED_E_ARG, "%s: unknown rounding %d", fn, rounding);
  if (R <= 0 || R > seed::kMaxCap)
    return fail(SEED_E_SHAPE, "%s: need 0 < R <= %d (got %d)", fn, seed::kMaxCap, R);
  SEED_PTR(U);
  SEED_PTR(V);
  SEED_PTR(Uk);
  SEED_PTR(Vk);
  return device_status(
      fn, seed::launch_round_factors(store_fmt_of(store_dtype), batch * heads, R, d_k, d_v, U, V,
                                     static_cast<uint16_t*>(Uk), static_cast<uint16_t*>(Vk),
                                     rounding == SEED_ROUND_STOCHASTIC, epoch,
                                     (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32),
                                     static_cast<hipStream_t>(stream)));
}

size_t seed_handoff_head_bytes(int d_k, int d_v, int R, int store_dtype) {
  if (!supported_dims(d_k, d_v) || R <= 0 || R > seed::kMaxCap) return 0;
  if (store_dtype != SEED_F32 && store_dtype != SEED_BF16 && store_dtype != SEED_F16) return 0;
  const size_t fb = store_dtype == SEED_F32 ? 4 : 2;
  return 4 * (size_t)d_k + fb * (size_t)(d_k + d_v) * R;
}

}  // extern "C"

namespace {

seed_status handoff(const char* fn, bool pack, int batch, int heads, int d_k, int d_v, int cap,
                    int R, int store_dtype, int n_sel, const int* idx, float* a, void* U, void* V,
                    void* buf, void* stream) {
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  if (store_dtype != SEED_F32 && store_dtype != SEED_BF16 && store_dtype != SEED_F16)
    return fail(SEED_E_ARG, "%s: unknown store dtype %d", fn, store_dtype);
  if (R <= 0 || cap < R || n_sel < 0)
    return fail(SEED_E_SHAPE, "%s: need 0 < R <= cap and n_sel >= 0 (got R=%d cap=%d n_sel=%d)",
                fn, R, cap, n_sel);
  if (cap > seed::kMaxCap)
    return fail(SEED_E_UNSUPPORTED, "%s: capacity %d above %d", fn, cap, seed::kMaxCap);
  if ((long long)n_sel * heads > 0x7fffffffLL)
    return fail(SEED_E_SHAPE, "%s: n_sel * heads exceeds the grid limit", fn);
  if (n_sel == 0) return ok();
  SEED_PTR(idx);
  SEED_PTR(a);
  SEED_PTR(U);
  SEED_PTR(V);
  SEED_PTR(buf);
  return device_status(
      fn, seed::launch_handoff(pack, batch, heads, d_k, d_v, cap, R, store_dtype == SEED_F32 ? 4 : 2,
                               n_sel, idx, a, U, V, buf, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

seed_status seed_pack_states(int batch, int heads, int d_k, int d_v, int cap, int R,
                             int store_dtype, int n_sel, const int* sel, const float* a,
                             const void* U, const void* V, void* buf, void* stream) {
  return handoff("seed_pack_states", true, batch, heads, d_k, d_v, cap, R, store_dtype, n_sel, sel,
                 const_cast<float*>(a), const_cast<void*>(U), const_cast<void*>(V), buf, stream);
}

seed_status seed_unpack_states(int batch, int heads, int d_k, int d_v, int cap, int R,
                               int store_dtype, int n_sel, const int* slot, const void* buf,
                               float* a, void* U, void* V, void* stream) {
  return handoff("seed_unpack_states", false, batch, heads, d_k, d_v, cap, R, store_dtype, n_sel,
                 slot, a, U, V, const_cast<void*>(buf), stream);
}

seed_status seed_join_states(int rule, int batch, int heads, int d_k, int d_v, int cap, int R,
                             int r, int n_sel, const int* slot, const void* buf, float* a,
                             float* U, float* V, float* gam, void* stream) {
  const char* fn = "seed_join_states";
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  if (rule != SEED_RULE_GDN && rule != SEED_RULE_KDA && rule != SEED_RULE_MAMBA2)
    return fail(SEED_E_ARG, "%s: unknown rule %d", fn, rule);
  if (R <= 0 || r < R || r >= cap || n_sel < 0)
    return fail(SEED_E_SHAPE, "%s: need 0 < R <= r < cap and n_sel >= 0 (got R=%d r=%d cap=%d "
                "n_sel=%d)", fn, R, r, cap, n_sel);
  if (cap > seed::kMaxCap)
    return fail(SEED_E_UNSUPPORTED, "%s: capacity %d above %d", fn, cap, seed::kMaxCap);
  if ((long long)n_sel * heads > 0x7fffffffLL)
    return fail(SEED_E_SHAPE, "%s: n_sel * heads exceeds the grid limit", fn);
  if (n_sel == 0) return ok();
  SEED_PTR(slot);
  SEED_PTR(buf);
  SEED_PTR(a);
  SEED_PTR(U);
  SEED_PTR(V);
  if (gam != nullptr) SEED_PTR(gam);
  const int gam_len = gam == nullptr ? 0 : (rule == SEED_RULE_KDA ? d_k : 1);
  return device_status(fn, seed::launch_join(batch, heads, d_k, d_v, cap, R, r, gam_len, n_sel,
                                             slot, buf, a, U, V, gam,
                                             static_cast<hipStream_t>(stream)));
}

int seed_stat_fields(void) { return seed::stat_fields(); }

seed_status seed_state_stats(int batch, int heads, int d_k, int d_v, int R, const float* S,
                             const float* vbar, float* rec, float* spec_S, float* spec_C,
                             void* stream) {
  const char* fn = "seed_state_stats";
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  if (R < 0 || R > d_k)
    return fail(SEED_E_SHAPE, "%s: need 0 <= R <= d_k (got %d)", fn, R);
  SEED_PTR(S);
  SEED_PTR(vbar);
  SEED_PTR(rec);
  if (spec_S != nullptr) SEED_PTR(spec_S);
  if (spec_C != nullptr) SEED_PTR(spec_C);
  if (seed::stats_lds_bytes(d_k, 1) > seed::kMaxLds)
    return fail(SEED_E_UNSUPPORTED, "%s: d_k=%d needs more LDS than a CU has", fn, d_k);
  return device_status(fn, seed::launch_state_stats(batch, heads, d_k, d_v, R, S, vbar, rec,
                                                    spec_S, spec_C,
                                                    static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

seed_status check_sched(const char* fn, int rule, int batch, int heads, int d_k, int d_v, int R,
                        int W, int D) {
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  if (rule != SEED_RULE_GDN && rule != SEED_RULE_KDA && rule != SEED_RULE_MAMBA2)
    return fail(SEED_E_ARG, "%s: unknown rule %d", fn, rule);
  if (W <= 0 || D < 0 || D >= W)
    return fail(SEED_E_SHAPE, "%s: need W > 0 and 0 <= D < W (got W=%d D=%d)", fn, W, D);
  if (R != 16 && R != 32)
    return fail(SEED_E_UNSUPPORTED, "%s: built for R = 16 or 32 (got %d)", fn, R);
  if (R + W + D > seed::kMaxCap)
    return fail(SEED_E_UNSUPPORTED, "%s: R + W + D = %d above %d", fn, R + W + D, seed::kMaxCap);
  return SEED_OK;
}

}  // namespace

extern "C" {

seed_status seed_decode_step_sched(int rule, int batch, int heads, int d_k, int d_v, int R, int W,
                                   int D, int t, const int* t_start, float* a, float* KU,
                                   float* KV, float* Uw, float* Vw, float* gam, float* gam_snap,
                                   const float* vbar, const void* q, const void* k,
                                   const void* v, int in_dtype, const float* g, const float* beta,
                                   float* o, void* stream) {
  const char* fn = "seed_decode_step_sched";
  seed_status st = check_sched(fn, rule, batch, heads, d_k, d_v, R, W, D);
  if (st != SEED_OK) return st;
  st = check_step_inputs(fn, rule, q, k, v, in_dtype, g, beta, o);
  if (st != SEED_OK) return st;
  SEED_PTR(t_start);
  SEED_PTR(a);
  SEED_PTR(KU);
  SEED_PTR(KV);
  SEED_PTR(Uw);
  SEED_PTR(Vw);
  SEED_PTR(gam);
  SEED_PTR(gam_snap);
  SEED_PTR(vbar);
  const seed::RingArgs ring{t_start, t, W, D, KU, KV, gam_snap};
  return device_status(
      fn, seed::launch_step(rule, in_dtype == SEED_BF16, seed::kStoreRing, batch, heads, d_k, d_v,
                            W + D, R + W + D - 1, R, a, Uw, Vw, nullptr, nullptr, gam, vbar, q, k,
                            v, g, beta, o, static_cast<hipStream_t>(stream), &ring));
}

seed_status seed_compress_sched(int rule, int batch, int heads, int d_k, int d_v, int R, int W,
                                int D, int t_snap, const int* t_start, int n_units,
                                const int* units, float* KU, float* KV, const float* Uw,
                                const float* Vw, const float* gam_snap, void* stream) {
  const char* fn = "seed_compress_sched";
  seed_status st = check_sched(fn, rule, batch, heads, d_k, d_v, R, W, D);
  if (st != SEED_OK) return st;
  if (n_units < 0 || (long long)n_units > (long long)batch * heads)
    return fail(SEED_E_SHAPE, "%s: need 0 <= n_units <= batch * heads (got %d)", fn, n_units);
  if (n_units == 0) return ok();
  SEED_PTR(t_start);
  SEED_PTR(units);
  SEED_PTR(KU);
  SEED_PTR(KV);
  SEED_PTR(Uw);
  SEED_PTR(Vw);
  SEED_PTR(gam_snap);
  if (seed::compress_lds_bytes(R + W, R) > seed::kMaxLds)
    return fail(SEED_E_UNSUPPORTED, "%s: %d columns at rank %d need more LDS than a CU has", fn,
                R + W, R);
  seed::CompressArgs args{};
  args.units = n_units;
  args.cap = W + D;
  args.n = R + W;
  args.R = R;
  args.U = const_cast<float*>(Uw);
  args.V = const_cast<float*>(Vw);
  args.gam = const_cast<float*>(gam_snap);
  args.gam_per_row = rule == SEED_RULE_KDA;
  args.list = units;
  args.t_start = t_start;
  args.heads = heads;
  args.t_snap = t_snap;
  args.W = W;
  args.D = D;
  args.units_total = batch * heads;
  args.KU = KU;
  args.KV = KV;
  return device_status(fn, seed::launch_compress(d_k, d_v, seed::kStoreRing, args,
                                                 static_cast<hipStream_t>(stream)));
}

seed_status seed_state_from_dense(int batch, int heads, int d_k, int d_v, int cap, int R,
                                  const float* S, const float* vbar, float* a, float* U,
                                  float* V, void* stream) {
  const char* fn = "seed_state_from_dense";
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  if (cap <= 0 || R <= 0 || R > cap || R > d_k || R > d_v)
    return fail(SEED_E_SHAPE, "%s: need 0 < R <= min(cap, d_k, d_v) (got R=%d cap=%d)", fn, R,
                cap);
  if (cap > seed::kMaxCap)
    return fail(SEED_E_UNSUPPORTED, "%s: capacity %d above %d", fn, cap, seed::kMaxCap);
  if (R > 32) return fail(SEED_E_UNSUPPORTED, "%s: rank %d above 32", fn, R);
  SEED_PTR(S);
  SEED_PTR(vbar);
  SEED_PTR(a);
  SEED_PTR(U);
  SEED_PTR(V);
  if (seed::convert_lds_bytes(d_k, R) > seed::kMaxLds)
    return fail(SEED_E_UNSUPPORTED, "%s: d_k=%d at rank %d needs more LDS than a CU has", fn, d_k,
                R);
  seed::CompressArgs args{};
  args.units = batch * heads;
  args.cap = cap;
  args.n = d_k;
  args.R = R;
  args.U = U;
  args.V = V;
  args.heads = heads;
  args.S = S;
  args.vbar = vbar;
  args.a = a;
  return device_status(fn, seed::launch_convert(d_k, d_v, args, static_cast<hipStream_t>(stream)));
}

seed_status dense_decode_step(int rule, int batch, int heads, int d_k, int d_v, float* S,
                              const void* q, const void* k, const void* v, int in_dtype,
                              const float* g, const float* beta, float* o, void* stream) {
  const char* fn = "dense_decode_step";
  seed_status st = check_units(fn, batch, heads, d_k, d_v);
  if (st != SEED_OK) return st;
  st = check_step_inputs(fn, rule, q, k, v, in_dtype, g, beta, o);
  if (st != SEED_OK) return st;
  SEED_PTR(S);
  return device_status(fn, seed::launch_dense(rule, in_dtype == SEED_BF16, batch, heads, d_k, d_v,
                                              S, q, k, v, g, beta, o,
                                              static_cast<hipStream_t>(stream)));
}

seed_status seed_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  const char* fn = "seed_stream_copy";
  SEED_PTR(src);
  SEED_PTR(dst);
  if (bytes % 16 != 0) return fail(SEED_E_ARG, "%s: bytes (%zu) must be a multiple of 16", fn, bytes);
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes)
    return fail(SEED_E_ARG, "%s: src and dst overlap", fn);
  return device_status(fn, seed::launch_stream_copy(src, dst, bytes,
                                                     static_cast<hipStream_t>(stream)));
}

size_t seed_workspace_bytes(int batch, int heads, int d_k, int d_v, int cap, int R) {
  const size_t reject = static_cast<size_t>(-1);
  if (batch <= 0 || heads <= 0 || (long long)batch * heads > 0x7fffffffLL) return reject;
  if (!supported_dims(d_k, d_v)) return reject;
  if (cap <= 0 || cap > seed::kMaxCap || R <= 0 || R > cap || R > 32) return reject;
  return 0;
}

const char* seed_status_string(int status) {
  switch (status) {
    case SEED_OK: return "ok";
    case SEED_E_ARG: return "invalid argument";
    case SEED_E_SHAPE: return "inconsistent shape";
    case SEED_E_UNSUPPORTED: return "unsupported shape";
    case SEED_E_FULL: return "factor capacity full";
    case SEED_E_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* seed_last_error(void) { return g_err; }

int seed_abi_version(void) { return 109; }

}  // extern "C"
