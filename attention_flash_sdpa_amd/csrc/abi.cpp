// Host side of the C ABI declared in include/sdpa.h: argument validation,
// workspace planning and kernel selection.  Validation happens before any
// HIP call, so argument errors need no GPU and leave outputs untouched.
#include "sdpa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;
thread_local const char* g_last_kernel = "";
std::atomic<int64_t> g_num_splits{0};
std::atomic<int64_t> g_relpos_fused{1};
std::atomic<int64_t> g_split64{1};
std::atomic<int64_t> g_split64w{1};
std::atomic<int64_t> g_tiled{1};
std::atomic<int64_t> g_generic_waves{0};
std::atomic<int64_t> g_relpos_mfma{1};
std::atomic<int64_t> g_tgrad_mfma{1};
std::atomic<int64_t> g_bwd_concurrent{1};

// The tuning knobs as one call sees them: read once at the call's start, so
// the route, the split count and the workspace check of that call agree even
// if another thread changes a knob meanwhile.
struct Tuning {
  int64_t num_splits, relpos_fused, split64, split64w, tiled, generic_waves;
};
Tuning tuning_now() {
  return {g_num_splits.load(), g_relpos_fused.load(), g_split64.load(), g_split64w.load(), g_tiled.load(),
          g_generic_waves.load()};
}

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool dtype_ok(int d) { return d == SDPA_F32 || d == SDPA_BF16 || d == SDPA_F16; }
bool is16(int d) { return d == SDPA_BF16 || d == SDPA_F16; }

void set_strides(int layout, int64_t H, int64_t T, int64_t D, int64_t* sb, int64_t* sh, int64_t* st) {
  if (layout == SDPA_BHSD) { *sb = H * T * D; *sh = T * D; *st = D; }
  else { *sb = T * H * D; *sh = D; *st = H * D; }
}

// Split-KV chunk count: few query rows against a long key range leave most of
// the GPU idle, so the key range is cut into chunks that run in parallel and
// are merged by their log-sum-exp afterwards.  The count depends on sizes and
// knobs only (not on the mask), so sdpa_workspace_size can answer before the
// call; a call whose route cannot split runs unsplit (fwd_prepare).
int plan_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D, int dtype, const Tuning& tu) {
  if (!sdpa::kSplitKvBuilt || !is16(dtype)) return 1;
  const int64_t forced = tu.num_splits;
  if (D == 16) {
    // the head_dim-16 query-packed kernel (few queries)
    if (Tq > 8) return 1;
    if (forced >= 1) return (int)std::min<int64_t>(forced, std::max<int64_t>(1, (Tkv + 63) / 64));
    // one wave per (4 heads, 8 queries, key chunk): aim at ~512 waves with
    // chunks of >= 64 keys (two tiles: the loads of the second overlap the first)
    const int64_t waves = B * ((Hq + 3) / 4) * ((Tq + 7) / 8);
    if (waves >= 512 || Tkv <= 64) return 1;
    int64_t s = (512 + waves - 1) / waves;
    s = std::min<int64_t>(s, (Tkv + 63) / 64);
    return (int)std::max<int64_t>(1, std::min<int64_t>(s, 1024));
  }
  if ((D != 64 && D != 128) || !tu.tiled) return 1;
  // the double-buffered head_dim 64 / 128 kernel: up to 64 chunks of >= 32 keys
  if (forced >= 1) return (int)std::min<int64_t>({forced, 64, std::max<int64_t>(1, (Tkv + 31) / 32)});
  // workgroups of 4 waves x 32 query rows (heads sharing a KV head packed
  // together): under 128 of them leave the 256 CUs mostly idle; aim at ~512
  // with chunks of >= 256 keys (8 tiles: the pipeline's fill is paid once per chunk)
  const int64_t grp = Hq / std::max<int64_t>(Hkv, 1);
  const int64_t hpw = grp % 4 == 0 ? 4 : grp % 2 == 0 ? 2 : 1;
  const int64_t wgs = B * (Hq / hpw) * ((Tq + 32 * (4 / hpw) - 1) / (32 * (4 / hpw)));
  if (wgs >= 128 || Tkv < 512) return 1;
  const int64_t s = std::min<int64_t>({(512 + wgs - 1) / wgs, Tkv / 256, 64});
  return (int)std::max<int64_t>(1, s);
}

size_t split_bytes(int splits, int64_t B, int64_t Hq, int64_t Tq, int64_t D) {
  if (splits <= 1) return 0;
  return align256((size_t)splits * B * Hq * Tq * D * 4) + align256((size_t)splits * B * Hq * Tq * 2 * 4);
}

size_t terms_bytes(int64_t B, int64_t H, int64_t T, int64_t gh, int64_t gw) {
  return align256((size_t)B * H * T * gh * 4) + align256((size_t)B * H * T * gw * 4);
}

// Largest tensor, in elements, that a call may describe: 2^40 elements is
// several times the memory of any one device, and keeps every element offset
// the kernels and the workspace planning form far from 64-bit overflow.
constexpr int64_t kMaxElements = int64_t(1) << 40;

// True if the product of the positive factors is at most kMaxElements
// (checked factor by factor, so the product itself never overflows).
bool elements_ok(std::initializer_list<int64_t> factors) {
  int64_t acc = 1;
  for (int64_t f : factors) {
    if (f <= 0 || acc > kMaxElements / f) return false;
    acc *= f;
  }
  return true;
}

int check_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tkv <= 0 || D <= 0)
    return fail(SDPA_ERR_INVALID, "all sizes must be positive (B=%lld Hq=%lld Hkv=%lld Tq=%lld Tkv=%lld D=%lld)",
                (long long)B, (long long)Hq, (long long)Hkv, (long long)Tq, (long long)Tkv, (long long)D);
  if (Hq % Hkv) return fail(SDPA_ERR_INVALID, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (Tq > INT32_MAX || Tkv > INT32_MAX || B > 65535 || Hq > 65535)
    return fail(SDPA_ERR_UNSUPPORTED, "sizes beyond the launch grid limits");
  if (!elements_ok({B, Hq, Tq, D}) || !elements_ok({B, Hkv, Tkv, D}) || !elements_ok({B, Hq, Tq, Tkv}))
    return fail(SDPA_ERR_UNSUPPORTED, "tensors of more than 2^40 elements are beyond device memory");
  return SDPA_OK;
}

int check_dtypes(int dtype, int out_dtype, int layout, int64_t D) {
  if (!dtype_ok(dtype)) return fail(SDPA_ERR_INVALID, "unknown dtype %d", dtype);
  if (!dtype_ok(out_dtype) || (out_dtype != dtype && out_dtype != SDPA_F32))
    return fail(SDPA_ERR_INVALID, "out_dtype must equal dtype or be SDPA_F32");
  if (layout != SDPA_BSHD && layout != SDPA_BHSD) return fail(SDPA_ERR_INVALID, "unknown layout %d", layout);
  if (D > 128) return fail(SDPA_ERR_UNSUPPORTED, "head_dim %lld > 128 is not built", (long long)D);
  if (is16(dtype) && D != 16 && D != 32 && D != 64 && D != 128)
    return fail(SDPA_ERR_UNSUPPORTED, "16-bit head_dim must be 16, 32, 64 or 128 (got %lld)", (long long)D);
  return SDPA_OK;
}

sdpa::FwdParams base_params(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype,
                            int layout, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D,
                            float scale, float* lse) {
  sdpa::FwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.dtype = dtype; p.out_dtype = out_dtype;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Tq = Tq; p.Tkv = Tkv; p.D = D;
  set_strides(layout, Hq, Tq, D, &p.q_sb, &p.q_sh, &p.q_st);
  set_strides(layout, Hkv, Tkv, D, &p.k_sb, &p.k_sh, &p.k_st);
  p.scale = std::isnan(scale) ? (float)(1.0 / std::sqrt((double)D)) : scale;
  p.bias = sdpa::BIAS_NONE;
  p.num_splits = 1;
  return p;
}

// Mask argument -> bias fields of the kernel parameters (FwdParams or BwdParams).
template <class P>
int apply_mask(const sdpa_mask* mask, P& p) {
  if (!mask || mask->kind == SDPA_MASK_NONE) return SDPA_OK;
  switch (mask->kind) {
    case SDPA_MASK_CAUSAL:
      p.bias = sdpa::BIAS_CAUSAL;
      p.offset = mask->offset;
      return SDPA_OK;
    case SDPA_MASK_SLIDING:
      if (mask->window < 1) return fail(SDPA_ERR_INVALID, "sliding window must be >= 1 (got %lld)", (long long)mask->window);
      p.bias = sdpa::BIAS_SLIDING;
      p.offset = mask->offset;
      p.window = mask->window;
      return SDPA_OK;
    case SDPA_MASK_ADDITIVE:
    case SDPA_MASK_BOOL:
      if (!mask->data) return fail(SDPA_ERR_INVALID, "tensor mask needs a data pointer");
      if (mask->kind == SDPA_MASK_ADDITIVE && mask->data_dtype != SDPA_F32 && mask->data_dtype != SDPA_BF16)
        return fail(SDPA_ERR_INVALID, "additive mask dtype must be SDPA_F32 or SDPA_BF16");
      for (int a = 0; a < 4; ++a)
        if (mask->stride[a] < 0) return fail(SDPA_ERR_INVALID, "mask strides must be >= 0");
      p.bias = mask->kind == SDPA_MASK_ADDITIVE ? sdpa::BIAS_ADDITIVE : sdpa::BIAS_BOOL;
      p.mdata = mask->data;
      p.mdtype = mask->data_dtype;
      for (int a = 0; a < 4; ++a) p.ms[a] = mask->stride[a];
      return SDPA_OK;
    default:
      return fail(SDPA_ERR_INVALID, "unknown mask kind %d", mask->kind);
  }
}

// Dropout rate -> (16-bit keep threshold, factor of a kept weight): keep iff
// the element's 16-bit uniform >= thresh, thresh = floor(rate * 65536 + 0.5)
// clamped to 65535, so the kept fraction is (65536 - thresh) / 65536 and the
// factor 65536 / (65536 - thresh) makes the dropped weights unbiased.
int dropout_plan(float rate, uint32_t* thresh, float* kscale) {
  if (!(rate >= 0.0f && rate < 1.0f)) return fail(SDPA_ERR_INVALID, "dropout rate must be in [0, 1) (got %g)", (double)rate);
  const double t = std::floor((double)rate * 65536.0 + 0.5);
  *thresh = (uint32_t)std::min(65535.0, t);
  *kscale = (float)(65536.0 / (65536.0 - (double)*thresh));
  return SDPA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

enum Route { R_GENERIC, R_D16, R_WINDOW, R_SPLIT64W, R_SPLIT64, R_TILED, R_MFMA };

// The kernel a call runs on: the first route whose conditions hold.
Route route_of(const sdpa::FwdParams& p, const Tuning& tu) {
  // The MFMA kernels take each row's running max on scores already multiplied
  // by scale, which needs scale > 0; other scales run on the generic kernel.
  if (!(p.scale > 0.0f && std::isfinite(p.scale))) return R_GENERIC;
  // Dropout runs on the double-buffered kernel (no mask, causal, sliding), else on the
  // general MFMA kernel where it applies, else on the generic one.
  if (p.keep) {
    if (tu.tiled && sdpa::tiled_supports(p)) return R_TILED;
    return sdpa::flash_mfma_supports(p) ? R_MFMA : R_GENERIC;
  }
  if (sdpa::d16_supports(p)) return R_D16;
  if (sdpa::window_supports(p)) return R_WINDOW;
  const int64_t wide = tu.split64w;     // 0 off, 1 where the shape fills the CUs, 2 wherever supported
  if (tu.split64 && wide && sdpa::split64w_supports(p, wide == 1)) return R_SPLIT64W;
  if (tu.split64 && sdpa::split64_supports(p)) return R_SPLIT64;
  if (tu.tiled && sdpa::tiled_supports(p)) return R_TILED;
  if (sdpa::flash_mfma_supports(p)) return R_MFMA;
  return R_GENERIC;
}

int launch(const sdpa::FwdParams& p0, const Tuning& tu, hipStream_t s) {
  hipError_t e;
  const char* name;
  sdpa::FwdParams p = p0;
  p.generic_multiwave = tu.generic_waves != 1;
  switch (route_of(p, tu)) {
    case R_D16:
      name = p.Tq <= 8 ? "d16_qpack_kernel" : "d16_kpack_kernel";
      e = sdpa::launch_d16(p, s);
      break;
    case R_WINDOW: name = "flash_window_kernel"; e = sdpa::launch_window(p, s); break;
    case R_SPLIT64W: name = "flash_split64w_kernel"; e = sdpa::launch_split64w(p, s); break;
    case R_SPLIT64: name = "flash_split64_kernel"; e = sdpa::launch_split64(p, s); break;
    case R_TILED: name = "flash_tiled_kernel"; e = sdpa::launch_tiled(p, s); break;
    case R_MFMA: name = "flash_mfma_kernel"; e = sdpa::launch_flash_mfma(p, s); break;
    default: name = "generic_fwd_kernel"; e = sdpa::launch_generic_fwd(p, s); break;
  }
  g_last_kernel = name;
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

// True if the attention kernel a rel-pos call reaches without term arrays
// forms the terms itself (no relpos_terms launch): every MFMA route that
// accepts such a call does; the generic kernel does where the tables and the
// per-lane term rows fit its LDS.
bool relpos_fused_ok(const sdpa::FwdParams& p, const Tuning& tu) {
  if (!tu.relpos_fused) return false;
  sdpa::FwdParams q = p;
  q.term_h = nullptr;
  q.term_w = nullptr;
  if (route_of(q, tu) != R_GENERIC) return true;            // a matrix-core kernel forms the terms
  // Only the vector-ALU kernel could form them: where a matrix-core kernel
  // takes the call with precomputed terms (head_dim 128, grids other than the
  // fused kernels'), the terms kernel runs first instead.
  alignas(16) static float probe[4] = {};
  sdpa::FwdParams t = q;
  t.term_h = probe;
  t.term_w = probe;
  if (route_of(t, tu) != R_GENERIC) return false;
  return sdpa::generic_relpos_supported(q, true);
}

// Rel-pos limits of every route (the generic kernel's term staging, the terms kernel).
int check_relpos_grid(int64_t grid_h, int64_t grid_w, int64_t D) {
  if (D <= 0) return fail(SDPA_ERR_INVALID, "head_dim must be positive (got %lld)", (long long)D);
  if (grid_h > 1024 || grid_w > 1024 || D > 128 || (D + 1) * grid_w * 4 > 65536)
    return fail(SDPA_ERR_UNSUPPORTED, "grid %lldx%lld with head_dim %lld is not built", (long long)grid_h,
                (long long)grid_w, (long long)D);
  return SDPA_OK;
}

// Kernel parameters of a rel-pos call (no term arrays yet).
sdpa::FwdParams relpos_params(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype,
                              int layout, int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D,
                              const void* rel_pos_h, const void* rel_pos_w, float scale, float* lse) {
  const int64_t T = grid_h * grid_w;
  sdpa::FwdParams p = base_params(q, k, v, o, dtype, out_dtype, layout, B, H, H, T, T, D, scale, lse);
  p.bias = sdpa::BIAS_RELPOS;
  p.grid_h = (int)grid_h;
  p.grid_w = (int)grid_w;
  p.rel_h = rel_pos_h;
  p.rel_w = rel_pos_w;
  return p;
}

}  // namespace

extern "C" {

size_t sdpa_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D,
                           float scale, int relpos, int64_t grid_h, int64_t grid_w) {
  if (!dtype_ok(dtype) || check_sizes(B, Hq, Hkv, Tq, Tkv, D)) return (size_t)-1;
  const Tuning tu = tuning_now();
  if (relpos) {
    if (grid_h <= 0 || grid_w <= 0 || grid_h > 1024 || grid_w > 1024 || grid_h * grid_w != Tq || Tq != Tkv ||
        Hkv != Hq)
      return (size_t)-1;
    static const char dummy = 0;
    const sdpa::FwdParams p = relpos_params(&dummy, &dummy, &dummy, (void*)&dummy, dtype, dtype, SDPA_BHSD, B, Hq,
                                            grid_h, grid_w, D, &dummy, &dummy, scale, nullptr);
    return relpos_fused_ok(p, tu) ? 0 : terms_bytes(B, Hq, Tq, grid_h, grid_w);
  }
  return split_bytes(plan_splits(B, Hq, Hkv, Tq, Tkv, D, dtype, tu), B, Hq, Tq, D);
}

}  // extern "C"

namespace {

// Validation and kernel parameters shared by sdpa_fwd and sdpa_fwd_noalloc:
// *need is the split-KV scratch the call's route takes (0 = none).
int fwd_prepare(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype, int layout,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D, float scale,
                const sdpa_mask* mask, float* lse, const Tuning& tu, sdpa::FwdParams* out, size_t* need) {
  if (!q || !k || !v || !o) return fail(SDPA_ERR_INVALID, "q, k, v and o must be non-null");
  int st = check_sizes(B, Hq, Hkv, Tq, Tkv, D);
  if (st) return st;
  st = check_dtypes(dtype, out_dtype, layout, D);
  if (st) return st;
  sdpa::FwdParams p = base_params(q, k, v, o, dtype, out_dtype, layout, B, Hq, Hkv, Tq, Tkv, D, scale, lse);
  st = apply_mask(mask, p);
  if (st) return st;
  p.num_splits = plan_splits(B, Hq, Hkv, Tq, Tkv, D, dtype, tu);
  // only the head_dim-16 and double-buffered kernels split; a call that lands
  // elsewhere (e.g. a tensor mask at head_dim 64 / 128) runs unsplit
  if (p.num_splits > 1) {
    const Route r = route_of(p, tu);
    if (r != R_D16 && r != R_TILED) p.num_splits = 1;
  }
  *need = split_bytes(p.num_splits, B, Hq, Tq, D);
  *out = p;
  return SDPA_OK;
}

void set_split_buffers(sdpa::FwdParams& p, void* base) {
  p.part_o = (float*)base;
  p.part_ml = (float*)((char*)base + align256((size_t)p.num_splits * p.B * p.Hq * p.Tq * p.D * 4));
}

}  // namespace

extern "C" {

int sdpa_fwd(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype, int layout,
             int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D, float scale,
             const sdpa_mask* mask, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  const Tuning tu = tuning_now();
  sdpa::FwdParams p;
  size_t need = 0;
  int st = fwd_prepare(q, k, v, o, dtype, out_dtype, layout, B, Hq, Hkv, Tq, Tkv, D, scale, mask, lse, tu, &p, &need);
  if (st) return st;
  if (need) {
    if (!workspace || workspace_bytes < need)
      return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
    set_split_buffers(p, workspace);
  }
  return launch(p, tu, (hipStream_t)stream);
}

int sdpa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype, int layout,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D, float scale,
                     const sdpa_mask* mask, float* lse, void* stream) {
  g_last_error.clear();
  const Tuning tu = tuning_now();
  sdpa::FwdParams p;
  size_t need = 0;
  int st = fwd_prepare(q, k, v, o, dtype, out_dtype, layout, B, Hq, Hkv, Tq, Tkv, D, scale, mask, lse, tu, &p, &need);
  if (st) return st;
  if (need > sdpa::kNoAllocScratchBytes && tu.num_splits == 0) {
    // an automatic split count is lowered to what the fixed scratch holds
    while (p.num_splits > 1 && split_bytes(p.num_splits, B, Hq, Tq, D) > sdpa::kNoAllocScratchBytes) --p.num_splits;
    need = split_bytes(p.num_splits, B, Hq, Tq, D);
  }
  if (need) {
    if (need > sdpa::kNoAllocScratchBytes)
      return fail(SDPA_ERR_UNSUPPORTED, "split-KV partials of %zu bytes exceed the fixed %zu-byte scratch", need,
                  sdpa::kNoAllocScratchBytes);
    void* scratch = nullptr;
    const hipError_t e = sdpa::noalloc_scratch(&scratch);
    if (e != hipSuccess) return fail(SDPA_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(e));
    set_split_buffers(p, scratch);
  }
  return launch(p, tu, (hipStream_t)stream);
}

int relpos_terms(const void* q, int dtype, int layout, int64_t B, int64_t H, int64_t grid_h, int64_t grid_w,
                 int64_t D, const void* rel_pos_h, const void* rel_pos_w, float* term_h, float* term_w,
                 void* stream) {
  g_last_error.clear();
  if (!q || !rel_pos_h || !rel_pos_w || !term_h || !term_w)
    return fail(SDPA_ERR_INVALID, "q, tables and term outputs must be non-null");
  if (B <= 0 || H <= 0 || grid_h <= 0 || grid_w <= 0 || D <= 0) return fail(SDPA_ERR_INVALID, "all sizes must be positive");
  if (!dtype_ok(dtype)) return fail(SDPA_ERR_INVALID, "unknown dtype %d", dtype);
  if (layout != SDPA_BSHD && layout != SDPA_BHSD) return fail(SDPA_ERR_INVALID, "unknown layout %d", layout);
  if (D > 128 || grid_h > 1024 || grid_w > 1024 || (D + 1) * grid_w * 4 > 65536)
    return fail(SDPA_ERR_UNSUPPORTED, "grid %lldx%lld with head_dim %lld is not built", (long long)grid_h,
                (long long)grid_w, (long long)D);
  if (B > 65535 || H > 65535) return fail(SDPA_ERR_UNSUPPORTED, "sizes beyond the launch grid limits");
  if (!elements_ok({B, H, grid_h * grid_w, grid_h + grid_w}))
    return fail(SDPA_ERR_UNSUPPORTED, "term arrays of more than 2^40 elements are beyond device memory");
  sdpa::TermsParams t;
  t.q = q; t.dtype = dtype; t.B = B; t.H = H; t.T = grid_h * grid_w; t.D = D;
  set_strides(layout, H, t.T, D, &t.q_sb, &t.q_sh, &t.q_st);
  t.rel_h = rel_pos_h; t.rel_w = rel_pos_w;
  t.grid_h = (int)grid_h; t.grid_w = (int)grid_w;
  t.term_h = term_h; t.term_w = term_w;
  t.use_mfma = g_relpos_mfma.load() != 0;
  hipError_t e = sdpa::launch_relpos_terms(t, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "relpos_terms launch failed: %s", hipGetErrorString(e));
  return SDPA_OK;
}

int sdpa_relpos_fwd(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype, int layout,
                    int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D, const void* rel_pos_h,
                    const void* rel_pos_w, float scale, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !rel_pos_h || !rel_pos_w)
    return fail(SDPA_ERR_INVALID, "q, k, v, o and both tables must be non-null");
  if (grid_h <= 0 || grid_w <= 0) return fail(SDPA_ERR_INVALID, "grid sizes must be positive");
  int st = check_relpos_grid(grid_h, grid_w, D);
  if (st) return st;
  const int64_t T = grid_h * grid_w;
  st = check_sizes(B, H, H, T, T, D);
  if (st) return st;
  st = check_dtypes(dtype, out_dtype, layout, D);
  if (st) return st;
  sdpa::FwdParams p = relpos_params(q, k, v, o, dtype, out_dtype, layout, B, H, grid_h, grid_w, D, rel_pos_h,
                                    rel_pos_w, scale, lse);
  const Tuning tu = tuning_now();
  // The fused route forms the terms inside the attention kernel: no workspace.
  if (relpos_fused_ok(p, tu)) return launch(p, tu, (hipStream_t)stream);
  const size_t need = terms_bytes(B, H, T, grid_h, grid_w);
  if (!workspace || workspace_bytes < need)
    return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  float* th = (float*)workspace;
  float* tw = (float*)((char*)workspace + align256((size_t)B * H * T * grid_h * 4));
  st = relpos_terms(q, dtype, layout, B, H, grid_h, grid_w, D, rel_pos_h, rel_pos_w, th, tw, stream);
  if (st) return st;
  p.term_h = th;
  p.term_w = tw;
  return launch(p, tu, (hipStream_t)stream);
}

size_t sdpa_relpos_fwd_dropout_workspace_size(int64_t B, int64_t H, int64_t grid_h, int64_t grid_w) {
  if (grid_h <= 0 || grid_w <= 0 || grid_h > 1024 || grid_w > 1024) return (size_t)-1;
  if (!elements_ok({B, H, grid_h * grid_w, grid_h + grid_w})) return (size_t)-1;
  return terms_bytes(B, H, grid_h * grid_w, grid_h, grid_w);
}

int sdpa_relpos_fwd_dropout(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype, int layout,
                            int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D, const void* rel_pos_h,
                            const void* rel_pos_w, float scale, const uint32_t* keep, float rate, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !rel_pos_h || !rel_pos_w || !keep)
    return fail(SDPA_ERR_INVALID, "q, k, v, o, both tables and keep must be non-null");
  if (grid_h <= 0 || grid_w <= 0) return fail(SDPA_ERR_INVALID, "grid sizes must be positive");
  int st = check_relpos_grid(grid_h, grid_w, D);
  if (st) return st;
  const int64_t T = grid_h * grid_w;
  st = check_sizes(B, H, H, T, T, D);
  if (st) return st;
  st = check_dtypes(dtype, out_dtype, layout, D);
  if (st) return st;
  uint32_t thresh;
  float kscale;
  st = dropout_plan(rate, &thresh, &kscale);
  if (st) return st;
  sdpa::FwdParams p = relpos_params(q, k, v, o, dtype, out_dtype, layout, B, H, grid_h, grid_w, D, rel_pos_h,
                                    rel_pos_w, scale, lse);
  // The terms always go through the workspace: the kernels that take dropout
  // with the rel-pos bias read them from there.
  const size_t need = terms_bytes(B, H, T, grid_h, grid_w);
  if (!workspace || workspace_bytes < need)
    return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  float* th = (float*)workspace;
  float* tw = (float*)((char*)workspace + align256((size_t)B * H * T * grid_h * 4));
  st = relpos_terms(q, dtype, layout, B, H, grid_h, grid_w, D, rel_pos_h, rel_pos_w, th, tw, stream);
  if (st) return st;
  p.term_h = th;
  p.term_w = tw;
  p.keep = keep;
  p.keep_words = (T + 31) / 32;
  p.keep_scale = kscale;
  return launch(p, tuning_now(), (hipStream_t)stream);
}

int sdpa_relpos_fused(int dtype, int64_t D, int64_t grid_h, int64_t grid_w) {
  if (grid_h <= 0 || grid_w <= 0 || D <= 0 || !dtype_ok(dtype) || grid_h > 1024 || grid_w > 1024 || D > 128) return 0;
  static const char dummy = 0;
  const sdpa::FwdParams p = relpos_params(&dummy, &dummy, &dummy, (void*)&dummy, dtype, dtype, SDPA_BHSD, 1, 1,
                                          grid_h, grid_w, D, &dummy, &dummy, 1.0f, nullptr);
  return relpos_fused_ok(p, tuning_now()) ? 1 : 0;
}

int sdpa_dropout_mask(uint64_t seed, uint32_t step, float rate, int64_t B, int64_t Hq, int64_t Tq, int64_t Tkv,
                      uint32_t* keep, void* stream) {
  g_last_error.clear();
  if (!keep) return fail(SDPA_ERR_INVALID, "keep must be non-null");
  if (B <= 0 || Hq <= 0 || Tq <= 0 || Tkv <= 0) return fail(SDPA_ERR_INVALID, "all sizes must be positive");
  if (Tq > INT32_MAX || Tkv > INT32_MAX || B > INT32_MAX || Hq > INT32_MAX || B * Hq > INT32_MAX)
    return fail(SDPA_ERR_UNSUPPORTED, "sizes beyond the generator's 32-bit counter words");
  if (!elements_ok({B, Hq, Tq, (Tkv + 31) / 32}))
    return fail(SDPA_ERR_UNSUPPORTED, "keep-bit array of more than 2^40 words is beyond device memory");
  sdpa::DropoutParams d;
  float kscale;
  int st = dropout_plan(rate, &d.thresh, &kscale);
  if (st) return st;
  d.seed = seed;
  d.step = step;
  d.B = B; d.Hq = Hq; d.Tq = Tq; d.Tkv = Tkv;
  d.keep_words = (Tkv + 31) / 32;
  d.keep = keep;
  hipError_t e = sdpa::launch_dropout_mask(d, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "dropout mask launch failed: %s", hipGetErrorString(e));
  g_last_kernel = "dropout_mask_kernel";
  return SDPA_OK;
}

int sdpa_fwd_dropout(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype, int layout,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D, float scale,
                     const sdpa_mask* mask, const uint32_t* keep, float rate, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !keep) return fail(SDPA_ERR_INVALID, "q, k, v, o and keep must be non-null");
  int st = check_sizes(B, Hq, Hkv, Tq, Tkv, D);
  if (st) return st;
  st = check_dtypes(dtype, out_dtype, layout, D);
  if (st) return st;
  uint32_t thresh;
  float kscale;
  st = dropout_plan(rate, &thresh, &kscale);
  if (st) return st;
  sdpa::FwdParams p = base_params(q, k, v, o, dtype, out_dtype, layout, B, Hq, Hkv, Tq, Tkv, D, scale, lse);
  st = apply_mask(mask, p);
  if (st) return st;
  p.keep = keep;
  p.keep_words = (Tkv + 31) / 32;
  p.keep_scale = kscale;
  (void)workspace;
  (void)workspace_bytes;
  return launch(p, tuning_now(), (hipStream_t)stream);
}

size_t sdpa_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Tq) {
  if (!elements_ok({B, Hq, Tq})) return (size_t)-1;
  return align256((size_t)B * Hq * Tq * 4);
}

int sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int dtype, int o_dtype, int grad_dtype, int layout,
             int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D, float scale,
             const sdpa_mask* mask, const uint32_t* keep, float rate, void* workspace, size_t workspace_bytes,
             void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(SDPA_ERR_INVALID, "q, k, v, o, dout, lse, dq, dk and dv must be non-null");
  int st = check_sizes(B, Hq, Hkv, Tq, Tkv, D);
  if (st) return st;
  st = check_dtypes(dtype, o_dtype, layout, D);
  if (st) return st;
  if (grad_dtype != dtype && grad_dtype != SDPA_F32) return fail(SDPA_ERR_INVALID, "grad_dtype must equal dtype or be SDPA_F32");
  sdpa::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse; p.dq = dq; p.dk = dk; p.dv = dv;
  p.dtype = dtype; p.o_dtype = o_dtype; p.grad_dtype = grad_dtype;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Tq = Tq; p.Tkv = Tkv; p.D = D;
  set_strides(layout, Hq, Tq, D, &p.q_sb, &p.q_sh, &p.q_st);
  set_strides(layout, Hkv, Tkv, D, &p.k_sb, &p.k_sh, &p.k_st);
  p.scale = std::isnan(scale) ? (float)(1.0 / std::sqrt((double)D)) : scale;
  if (!std::isfinite(p.scale)) return fail(SDPA_ERR_INVALID, "scale must be finite");
  st = apply_mask(mask, p);
  if (st) return st;
  if (keep) {
    uint32_t thresh;
    st = dropout_plan(rate, &thresh, &p.keep_scale);
    if (st) return st;
    p.keep = keep;
    p.keep_words = (Tkv + 31) / 32;
  }
  if (!sdpa::bwd_supports(p))
    return fail(SDPA_ERR_UNSUPPORTED, "the backward pass is built for bf16 / fp16 inputs with head_dim 32, 64 or 128");
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* x : ptrs)
    if (!aligned16(x)) return fail(SDPA_ERR_UNSUPPORTED, "the backward pass needs 16-byte aligned tensors");
  const size_t need = align256((size_t)B * Hq * Tq * 4);
  if (!workspace || workspace_bytes < need)
    return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  p.delta = (float*)workspace;
  p.concurrent = g_bwd_concurrent.load() != 0;
  hipError_t e = sdpa::launch_bwd(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  g_last_kernel = "bwd_dkdv_kernel";
  return SDPA_OK;
}

// Workspace of sdpa_relpos_bwd: delta | term_h | term_w | dterm_h | dterm_w | dq_acc | group_h | group_w.
size_t relpos_bwd_bytes(int64_t B, int64_t H, int64_t gh, int64_t gw, int64_t D, size_t* offs) {
  const int64_t T = gh * gw;
  const size_t sz[8] = {align256((size_t)B * H * T * 4),      align256((size_t)B * H * T * gh * 4),
                        align256((size_t)B * H * T * gw * 4), align256((size_t)B * H * T * gh * 4),
                        align256((size_t)B * H * T * gw * 4), align256((size_t)B * H * T * D * 4),
                        align256(std::max((size_t)sdpa::relpos_group_splits(B * H * gw, gh) * gh * gh * D * 4,
                                          (size_t)sdpa::relpos_tgrad_wgs(B, H, gh, gw) * 128 * D * 4)),
                        align256(std::max((size_t)sdpa::relpos_group_splits(B * H * gh, gw) * gw * gw * D * 4,
                                          (size_t)sdpa::relpos_tgrad_wgs(B, H, gh, gw) * 128 * D * 4))};
  size_t tot = 0;
  for (int a = 0; a < 8; ++a) {
    if (offs) offs[a] = tot;
    tot += sz[a];
  }
  return tot;
}

size_t sdpa_relpos_bwd_workspace_size(int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D) {
  if (grid_h <= 0 || grid_w <= 0 || grid_h > 1024 || grid_w > 1024 || D <= 0 || D > 128) return (size_t)-1;
  if (B > 65535 || H > 65535 || !elements_ok({B, H, grid_h * grid_w, grid_h * grid_w})) return (size_t)-1;
  return relpos_bwd_bytes(B, H, grid_h, grid_w, D, nullptr);
}

}  // extern "C"

namespace {

// The rel-pos backward with optional dropout keep bits (keep NULL: none).
int relpos_bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, float* d_rel_pos_h, float* d_rel_pos_w, int dtype, int o_dtype,
                    int grad_dtype, int layout, int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D,
                    const void* rel_pos_h, const void* rel_pos_w, float scale, const uint32_t* keep, float rate,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !d_rel_pos_h || !d_rel_pos_w || !rel_pos_h ||
      !rel_pos_w)
    return fail(SDPA_ERR_INVALID, "every tensor argument must be non-null");
  if (grid_h <= 0 || grid_w <= 0) return fail(SDPA_ERR_INVALID, "grid sizes must be positive");
  if (grid_h > 1024 || grid_w > 1024)
    return fail(SDPA_ERR_UNSUPPORTED, "grid %lldx%lld is not built", (long long)grid_h, (long long)grid_w);
  const int64_t T = grid_h * grid_w;
  int st = check_sizes(B, H, H, T, T, D);
  if (st) return st;
  st = check_dtypes(dtype, o_dtype, layout, D);
  if (st) return st;
  if (grad_dtype != dtype && grad_dtype != SDPA_F32) return fail(SDPA_ERR_INVALID, "grad_dtype must equal dtype or be SDPA_F32");
  sdpa::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse; p.dq = dq; p.dk = dk; p.dv = dv;
  p.dtype = dtype; p.o_dtype = o_dtype; p.grad_dtype = grad_dtype;
  p.B = B; p.Hq = H; p.Hkv = H; p.Tq = T; p.Tkv = T; p.D = D;
  set_strides(layout, H, T, D, &p.q_sb, &p.q_sh, &p.q_st);
  set_strides(layout, H, T, D, &p.k_sb, &p.k_sh, &p.k_st);
  p.scale = std::isnan(scale) ? (float)(1.0 / std::sqrt((double)D)) : scale;
  if (!std::isfinite(p.scale)) return fail(SDPA_ERR_INVALID, "scale must be finite");
  p.bias = sdpa::BIAS_RELPOS;
  p.grid_h = (int)grid_h;
  p.grid_w = (int)grid_w;
  p.rel_h = rel_pos_h;
  p.rel_w = rel_pos_w;
  p.drel_h = d_rel_pos_h;
  p.drel_w = d_rel_pos_w;
  if (keep) {
    uint32_t thresh;
    st = dropout_plan(rate, &thresh, &p.keep_scale);
    if (st) return st;
    p.keep = keep;
    p.keep_words = (T + 31) / 32;
  }
  if (!sdpa::bwd_supports(p))
    return fail(SDPA_ERR_UNSUPPORTED, "the rel-pos backward is built for bf16 / fp16 inputs, head_dim 32, 64 or 128, "
                                      "grid_w >= 4 and grid_h + grid_w <= 128");
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* x : ptrs)
    if (!aligned16(x)) return fail(SDPA_ERR_UNSUPPORTED, "the backward pass needs 16-byte aligned tensors");
  size_t off[8];
  const size_t need = relpos_bwd_bytes(B, H, grid_h, grid_w, D, off);
  if (!workspace || workspace_bytes < need)
    return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  char* ws = (char*)workspace;
  p.delta = (float*)(ws + off[0]);
  float* th = (float*)(ws + off[1]);
  float* tw = (float*)(ws + off[2]);
  p.term_h = th;
  p.term_w = tw;
  p.dterm_h = (float*)(ws + off[3]);
  p.dterm_w = (float*)(ws + off[4]);
  p.dq_acc = (float*)(ws + off[5]);
  p.group_h = (float*)(ws + off[6]);
  p.group_w = (float*)(ws + off[7]);
  p.split_h = sdpa::relpos_group_splits(B * H * grid_w, grid_h);
  p.split_w = sdpa::relpos_group_splits(B * H * grid_h, grid_w);
  p.tgrad_mfma = g_tgrad_mfma.load() != 0;
  p.concurrent = g_bwd_concurrent.load() != 0;
  st = relpos_terms(q, dtype, layout, B, H, grid_h, grid_w, D, rel_pos_h, rel_pos_w, th, tw, stream);
  if (st) return st;
  const hipError_t e =
      sdpa::launch_bwd(p, (hipStream_t)stream, sdpa::launch_relpos_bwd_dq, sdpa::launch_relpos_bwd_tables);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "rel-pos backward launch failed: %s", hipGetErrorString(e));
  g_last_kernel = "bwd_dkdv_kernel";
  return SDPA_OK;
}

}  // namespace

extern "C" {

int sdpa_relpos_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, float* d_rel_pos_h, float* d_rel_pos_w, int dtype, int o_dtype,
                    int grad_dtype, int layout, int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D,
                    const void* rel_pos_h, const void* rel_pos_w, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return relpos_bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, d_rel_pos_h, d_rel_pos_w, dtype, o_dtype, grad_dtype,
                         layout, B, H, grid_h, grid_w, D, rel_pos_h, rel_pos_w, scale, nullptr, 0.0f, workspace,
                         workspace_bytes, stream);
}

int sdpa_relpos_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, float* d_rel_pos_h, float* d_rel_pos_w,
                            int dtype, int o_dtype, int grad_dtype, int layout, int64_t B, int64_t H, int64_t grid_h,
                            int64_t grid_w, int64_t D, const void* rel_pos_h, const void* rel_pos_w, float scale,
                            const uint32_t* keep, float rate, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!keep) {
    g_last_error.clear();
    return fail(SDPA_ERR_INVALID, "keep must be non-null");
  }
  return relpos_bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, d_rel_pos_h, d_rel_pos_w, dtype, o_dtype, grad_dtype,
                         layout, B, H, grid_h, grid_w, D, rel_pos_h, rel_pos_w, scale, keep, rate, workspace,
                         workspace_bytes, stream);
}

int sdpa_attention_weights(const void* q, const void* k, int dtype, int layout, int64_t B, int64_t Hq, int64_t Hkv,
                           int64_t Tq, int64_t Tkv, int64_t D, float scale, const sdpa_mask* mask, const float* lse,
                           const uint32_t* keep, float rate, float* weights, void* stream) {
  g_last_error.clear();
  if (!q || !k || !lse || !weights) return fail(SDPA_ERR_INVALID, "q, k, lse and weights must be non-null");
  int st = check_sizes(B, Hq, Hkv, Tq, Tkv, D);
  if (st) return st;
  st = check_dtypes(dtype, dtype, layout, D);
  if (st) return st;
  if (B * Hq > 65535 || (Tq + 63) / 64 > 65535) return fail(SDPA_ERR_UNSUPPORTED, "sizes beyond the launch grid limits");
  sdpa::FwdParams p = base_params(q, k, nullptr, nullptr, dtype, dtype, layout, B, Hq, Hkv, Tq, Tkv, D, scale,
                                  const_cast<float*>(lse));
  st = apply_mask(mask, p);
  if (st) return st;
  if (keep) {
    uint32_t thresh;
    st = dropout_plan(rate, &thresh, &p.keep_scale);
    if (st) return st;
    p.keep = keep;
    p.keep_words = (Tkv + 31) / 32;
  }
  hipError_t e = sdpa::launch_attn_weights(p, weights, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "attention weights launch failed: %s", hipGetErrorString(e));
  g_last_kernel = sdpa::attn_weights_mfma(p) ? "attn_weights_mfma_kernel" : "attn_weights_kernel";
  return SDPA_OK;
}

const char* sdpa_status_string(int status) {
  switch (status) {
    case SDPA_OK: return "ok";
    case SDPA_ERR_INVALID: return "invalid argument";
    case SDPA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SDPA_ERR_WORKSPACE: return "workspace too small";
    case SDPA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* sdpa_last_error(void) { return g_last_error.c_str(); }

const char* sdpa_last_kernel(void) { return g_last_kernel; }

int sdpa_set_tuning(const char* key, int64_t value) {
  g_last_error.clear();
  if (!key) return fail(SDPA_ERR_INVALID, "null key");
  if (!std::strcmp(key, "num_splits")) {
    if (value < 0 || value > 1024) return fail(SDPA_ERR_INVALID, "num_splits must be in [0, 1024]");
    g_num_splits.store(value);
    return SDPA_OK;
  }
  if (!std::strcmp(key, "split_halves")) {
    if (value != 0 && value != 1) return fail(SDPA_ERR_INVALID, "split_halves must be 0 or 1");
    g_split64.store(value);
    return SDPA_OK;
  }
  if (!std::strcmp(key, "split_wide")) {
    if (value < 0 || value > 2) return fail(SDPA_ERR_INVALID, "split_wide must be 0, 1 or 2");
    g_split64w.store(value);
    return SDPA_OK;
  }
  if (!std::strcmp(key, "relpos_mfma")) {
    if (value != 0 && value != 1) return fail(SDPA_ERR_INVALID, "relpos_mfma must be 0 or 1");
    g_relpos_mfma.store(value);
    return SDPA_OK;
  }
  if (!std::strcmp(key, "relpos_bwd_mfma")) {
    if (value != 0 && value != 1) return fail(SDPA_ERR_INVALID, "relpos_bwd_mfma must be 0 or 1");
    g_tgrad_mfma.store(value);
    return SDPA_OK;
  }
  if (!std::strcmp(key, "bwd_concurrent")) {
    if (value != 0 && value != 1) return fail(SDPA_ERR_INVALID, "bwd_concurrent must be 0 or 1");
    g_bwd_concurrent.store(value);
    return SDPA_OK;
  }
  if (!std::strcmp(key, "generic_waves")) {
    if (value != 0 && value != 1) return fail(SDPA_ERR_INVALID, "generic_waves must be 0 (automatic) or 1");
    g_generic_waves.store(value);
    return SDPA_OK;
  }
  if (!std::strcmp(key, "tiled")) {
    if (value != 0 && value != 1) return fail(SDPA_ERR_INVALID, "tiled must be 0 or 1");
    g_tiled.store(value);
    return SDPA_OK;
  }
  if (!std::strcmp(key, "relpos_fused")) {
    if (value != 0 && value != 1) return fail(SDPA_ERR_INVALID, "relpos_fused must be 0 or 1");
    g_relpos_fused.store(value);
    return SDPA_OK;
  }
  return fail(SDPA_ERR_INVALID, "unknown tuning key '%s'", key);
}

}  // extern "C"
