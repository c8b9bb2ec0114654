// vq_api.cpp -- the C ABI (include/vq.h): host-side validation, dispatch and
// error reporting.  Nothing here touches device memory; every check runs
// before anything is enqueued, so a rejected call leaves outputs untouched.
//
// The loud-failure rule for sliced codebooks follows the model card
// "Qwen3.8-27B-VQ-4.5bpw", Multi-machine (exo) note: a codebook that is not
// whole must be refused with an explanation, never read as if it were.

#include "vq.h"
#include "vq_kernels.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_err;

vq_status fail(vq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

// Largest buffer a kernel addresses with 32-bit offsets (2 GiB - 1).
constexpr int64_t kMaxBufferBytes = 0x7fffffff;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int32_t words_per_row(int32_t cols, int32_t d, int32_t log2_k) {
  if (cols <= 0 || (d != 2 && d != 4 && d != 8) || log2_k < vqmi::kMinBits || log2_k > vqmi::kMaxBits) return -1;
  const int64_t n_codes = cols / d;
  const int64_t blocks = (n_codes + 31) / 32;
  return (int32_t)(blocks * log2_k);
}

// Validates the tensor descriptor and fills `v`.
vq_status check_tensor(const vq_tensor* w, vqmi::TensorView* v) {
  if (!w) return fail(VQ_ERR_NULL, "tensor descriptor is NULL");
  if (!w->codes || !w->codebook || !w->scales)
    return fail(VQ_ERR_NULL, "tensor has a NULL pointer (codes=%p codebook=%p scales=%p)",
                (const void*)w->codes, (const void*)w->codebook, (const void*)w->scales);
  if ((w->d != 2 && w->d != 4 && w->d != 8) || w->log2_k < vqmi::kMinBits || w->log2_k > vqmi::kMaxBits ||
      (w->group != 64 && w->group != 128))
    return fail(VQ_ERR_GEOMETRY,
                "unsupported geometry d=%d log2_k=%d group=%d (supported: d in {2,4,8}, "
                "log2_k in [4, 14], group in {64,128})",
                w->d, w->log2_k, w->group);
  if (w->rows < 1 || w->cols < 1)
    return fail(VQ_ERR_SHAPE, "rows=%d cols=%d must be positive", w->rows, w->cols);
  if (w->group % w->d != 0)
    return fail(VQ_ERR_SHAPE, "group=%d is not a multiple of d=%d", w->group, w->d);
  if (w->cols % w->group != 0)
    return fail(VQ_ERR_SHAPE, "cols=%d is not a multiple of group=%d", w->cols, w->group);
  if ((w->cols / w->d) % 32 != 0)
    return fail(VQ_ERR_SHAPE, "cols/d=%d is not a multiple of 32 (rows hold whole 32-code blocks)",
                w->cols / w->d);
  if (w->num_experts < 1) return fail(VQ_ERR_SHAPE, "num_experts=%d must be >= 1", w->num_experts);
  if (w->codebook_per_expert != 0 && w->codebook_per_expert != 1)
    return fail(VQ_ERR_SHAPE, "codebook_per_expert=%d must be 0 or 1", w->codebook_per_expert);
  const int64_t n_cb = w->codebook_per_expert ? w->num_experts : 1;
  const int64_t want = n_cb * ((int64_t)1 << w->log2_k) * w->d;
  if (w->codebook_elems != want)
    return fail(VQ_ERR_SHAPE,
                "codebook has %lld fp16 values but K*d%s = %lld: a sliced or partial codebook "
                "cannot be used (codebooks must be replicated whole, never split)",
                (long long)w->codebook_elems, w->codebook_per_expert ? "*E" : "", (long long)want);
  const int64_t want_words = (int64_t)w->num_experts * w->rows * words_per_row(w->cols, w->d, w->log2_k);
  if (w->code_words != want_words)
    return fail(VQ_ERR_SHAPE,
                "codes hold %lld words but E*rows*Wr = %lld (Wr = %d for cols=%d d=%d log2_k=%d): codes "
                "packed for another geometry, or a short buffer",
                (long long)w->code_words, (long long)want_words, words_per_row(w->cols, w->d, w->log2_k),
                w->cols, w->d, w->log2_k);
  const int64_t want_scales = (int64_t)w->num_experts * w->rows * (w->cols / w->group);
  if (w->scale_elems != want_scales)
    return fail(VQ_ERR_SHAPE, "scales hold %lld values but E*rows*cols/group = %lld",
                (long long)w->scale_elems, (long long)want_scales);
  const int64_t elems = (int64_t)w->num_experts * w->rows * (int64_t)w->cols;
  if (elems > ((int64_t)1 << 40))
    return fail(VQ_ERR_SHAPE, "tensor too large (%lld weights)", (long long)elems);
  // The kernels address one expert's codes and scales with 32-bit buffer offsets.
  const int64_t code_bytes = (int64_t)w->rows * words_per_row(w->cols, w->d, w->log2_k) * 4;
  const int64_t scale_bytes = (int64_t)w->rows * (w->cols / w->group) * 2;
  if (code_bytes > kMaxBufferBytes || scale_bytes > kMaxBufferBytes)
    return fail(VQ_ERR_SHAPE, "one expert's codes (%lld bytes) or scales (%lld bytes) exceed %lld bytes",
                (long long)code_bytes, (long long)scale_bytes, (long long)kMaxBufferBytes);
  if (!aligned(w->codes, 16)) return fail(VQ_ERR_ALIGN, "codes pointer is not 16-byte aligned");
  if (!aligned(w->codebook, 16)) return fail(VQ_ERR_ALIGN, "codebook pointer is not 16-byte aligned");
  if (!aligned(w->scales, 4)) return fail(VQ_ERR_ALIGN, "scales pointer is not 4-byte aligned");
  v->codes = w->codes;
  v->codebook = w->codebook;
  v->scales = w->scales;
  v->rows = w->rows;
  v->cols = w->cols;
  v->d = w->d;
  v->log2_k = w->log2_k;
  v->group = w->group;
  v->num_experts = w->num_experts;
  v->cb_per_expert = w->codebook_per_expert;
  v->wr = words_per_row(w->cols, w->d, w->log2_k);
  return VQ_OK;
}

vq_status check_xy(const void* x, const void* y, const char* yname) {
  if (!x) return fail(VQ_ERR_NULL, "x is NULL");
  if (!y) return fail(VQ_ERR_NULL, "%s is NULL", yname);
  if (!aligned(x, 16)) return fail(VQ_ERR_ALIGN, "x is not 16-byte aligned");
  if (!aligned(y, 16)) return fail(VQ_ERR_ALIGN, "%s is not 16-byte aligned", yname);
  return VQ_OK;
}

vq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return VQ_OK;
  return fail(VQ_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

// Largest input width the streaming GEMV covers in one pass over x; wider
// rows run in column slices that add into an fp32 y.
constexpr int32_t kGemvOnePassCols = 20480;

enum class Call { kGemv, kGemm, kMoeGemv, kMoeGemm };

// Validates an I/O descriptor (NULL = defaults) for a call on `w`.
vq_status check_io(const vq_io* io, const vq_tensor* w, Call call, vqmi::IoSpec* out) {
  *out = vqmi::IoSpec{};
  if (!io) return VQ_OK;
  const bool routed = call == Call::kMoeGemv || call == Call::kMoeGemm;
  if (io->x_dtype != VQ_DTYPE_F16 && io->x_dtype != VQ_DTYPE_BF16)
    return fail(VQ_ERR_SHAPE, "io->x_dtype=%d: x must be VQ_DTYPE_F16 or VQ_DTYPE_BF16", io->x_dtype);
  if (io->y_dtype != VQ_DTYPE_F32 && io->y_dtype != VQ_DTYPE_F16 && io->y_dtype != VQ_DTYPE_BF16)
    return fail(VQ_ERR_SHAPE, "io->y_dtype=%d is not a vq_dtype", io->y_dtype);
  if (io->epilogue != VQ_EPILOGUE_NONE && io->epilogue != VQ_EPILOGUE_SWIGLU && io->epilogue != VQ_EPILOGUE_COMBINE)
    return fail(VQ_ERR_SHAPE, "io->epilogue=%d is not a vq_epilogue", io->epilogue);
  if (io->reserved != 0) return fail(VQ_ERR_SHAPE, "io->reserved must be 0");
  if (io->epilogue == VQ_EPILOGUE_SWIGLU && w->rows % 2 != 0)
    return fail(VQ_ERR_SHAPE, "SWIGLU needs interleaved (gate, up) row pairs: rows=%d is odd", w->rows);
  if (io->epilogue == VQ_EPILOGUE_COMBINE) {
    if (!routed) return fail(VQ_ERR_SHAPE, "COMBINE applies to routed calls (vq_moe_*) only");
    if (io->y_dtype != VQ_DTYPE_F32)
      return fail(VQ_ERR_SHAPE, "COMBINE adds the slots into an fp32 y: y_dtype must be VQ_DTYPE_F32");
    if (!io->route_weights) return fail(VQ_ERR_NULL, "COMBINE needs route_weights");
    if (!aligned(io->route_weights, 4)) return fail(VQ_ERR_ALIGN, "route_weights is not 4-byte aligned");
  }
  const bool plain_f32 = io->y_dtype == VQ_DTYPE_F32 && io->epilogue != VQ_EPILOGUE_SWIGLU;
  if ((call == Call::kGemv || call == Call::kMoeGemv) && w->cols > kGemvOnePassCols && !plain_f32)
    return fail(VQ_ERR_SHAPE,
                "cols=%d: the streaming GEMV adds column slices above %d input features into an fp32 y, so "
                "it takes y_dtype F32 without SWIGLU there (use the GEMM entry point)",
                w->cols, kGemvOnePassCols);
  out->x_bf16 = io->x_dtype == VQ_DTYPE_BF16;
  out->y_kind = io->y_dtype == VQ_DTYPE_F32 ? vqmi::kOutF32 : io->y_dtype == VQ_DTYPE_F16 ? vqmi::kOutF16
                                                                                          : vqmi::kOutBF16;
  out->epi = io->epilogue == VQ_EPILOGUE_SWIGLU ? vqmi::kEpiSwiglu
             : io->epilogue == VQ_EPILOGUE_COMBINE ? vqmi::kEpiCombine : vqmi::kEpiNone;
  out->route_w = io->route_weights;
  return VQ_OK;
}

vq_status check_moe(const vq_tensor* w, const void* x, int32_t x_per_slot, const int32_t* ids,
                    int32_t T, int32_t top_k, const void* y, vqmi::TensorView* v) {
  vq_status st = check_tensor(w, v);
  if (st != VQ_OK) return st;
  if (T < 0) return fail(VQ_ERR_SHAPE, "T=%d must be >= 0", T);
  if (top_k < 1) return fail(VQ_ERR_SHAPE, "top_k=%d must be >= 1", top_k);
  if (x_per_slot != 0 && x_per_slot != 1)
    return fail(VQ_ERR_SHAPE, "x_per_slot=%d must be 0 or 1", x_per_slot);
  if ((int64_t)T * top_k > (1 << 30)) return fail(VQ_ERR_SHAPE, "T*top_k too large");
  const int64_t x_bytes = (int64_t)T * (x_per_slot ? top_k : 1) * w->cols * 2;
  if (x_bytes > kMaxBufferBytes)
    return fail(VQ_ERR_SHAPE, "x holds %lld bytes; at most %lld per call", (long long)x_bytes,
                (long long)kMaxBufferBytes);
  if (T == 0) return VQ_OK;
  st = check_xy(x, y, "y");
  if (st != VQ_OK) return st;
  if (!ids) return fail(VQ_ERR_NULL, "expert_ids is NULL");
  if (!aligned(ids, 4)) return fail(VQ_ERR_ALIGN, "expert_ids is not 4-byte aligned");
  return VQ_OK;
}

}  // namespace

extern "C" {

int32_t vq_words_per_row(int32_t cols, int32_t d, int32_t log2_k) {
  return words_per_row(cols, d, log2_k);
}

const char* vq_last_error(void) { return g_err.c_str(); }

const char* vq_status_name(vq_status s) {
  switch (s) {
    case VQ_OK: return "VQ_OK";
    case VQ_ERR_NULL: return "VQ_ERR_NULL";
    case VQ_ERR_GEOMETRY: return "VQ_ERR_GEOMETRY";
    case VQ_ERR_SHAPE: return "VQ_ERR_SHAPE";
    case VQ_ERR_ALIGN: return "VQ_ERR_ALIGN";
    case VQ_ERR_WORKSPACE: return "VQ_ERR_WORKSPACE";
    case VQ_ERR_HIP: return "VQ_ERR_HIP";
  }
  return "VQ_ERR_UNKNOWN";
}

vq_status vq_dequant(const vq_tensor* w, int32_t expert, uint16_t* w_out, void* stream) {
  vqmi::TensorView v;
  vq_status st = check_tensor(w, &v);
  if (st != VQ_OK) return st;
  if (expert < 0 || expert >= w->num_experts)
    return fail(VQ_ERR_SHAPE, "expert=%d outside [0, %d)", expert, w->num_experts);
  if (!w_out) return fail(VQ_ERR_NULL, "w_out is NULL");
  if (!aligned(w_out, 16)) return fail(VQ_ERR_ALIGN, "w_out is not 16-byte aligned");
  return hip_status(vqmi::launch_dequant(v, expert, w_out, (hipStream_t)stream), "vq_dequant launch");
}

// Largest token count for which the streaming GEMV beats the MFMA GEMM,
// measured on MI355X at the benchmark shapes: the GEMV reads every code once
// per grid slice, the GEMM once per 32- or 128-token tile, split along K to
// fill the GPU.  Where the matrix-core GEMV takes the call it wins up to the
// token count gemv_mf_max_tokens gives (16-token mode; 17408x5120 d = 4:
// 14.2, 15.1 and 20.9 us at T = 5, 8 and 16 against 17.9, 18.8 and 22.1 us
// for the GEMM; d = 2: 18.8 against 24.8 us at T = 16) and up to 4 tokens
// otherwise (12.6-13.1 us at T = 3-4 against 17.7-17.9 us).  Elsewhere small matrices and d = 8 keep a few tokens on the scalar
// GEMV, and the rest wins up to T = 2 (two tokens per slice; 17408x5120 and
// 5120x17408, d = 2 and 4: 15.9-18.6 us against 17.3-21.7 us for the GEMM).
static int gemv_token_limit(const vqmi::TensorView& v, const vqmi::IoSpec& io) {
  const int rows = v.rows * v.num_experts;  // a stack counts all its experts' rows
  const bool small = (int64_t)rows * v.cols <= (int64_t)16 << 20;
  const bool plain_out = io.epi == vqmi::kEpiNone && io.y_kind == vqmi::kOutF32;
  const int mf = vqmi::gemv_mf_max_tokens(rows, v.cols, v.d, vqmi::device_cus(), plain_out);
  if (mf > 4) return mf;
  if (mf == 4) return small ? 6 : 4;
  if (small) return 6;
  if (v.d == 8) return 4;
  return 2;
}

static vq_status dense_call(const vq_tensor* w, const vq_io* io, const void* x, int32_t T, void* y,
                           void* stream, bool gemv) {
  vqmi::TensorView v;
  vq_status st = check_tensor(w, &v);
  if (st != VQ_OK) return st;
  const char* name = gemv ? "vq_gemv" : "vq_gemm";
  if ((int64_t)w->num_experts * w->rows > (1 << 28))
    return fail(VQ_ERR_SHAPE, "%s: a stack of %d x %d rows is too large", name, w->num_experts, w->rows);
  vqmi::IoSpec ios;
  st = check_io(io, w, gemv ? Call::kGemv : Call::kGemm, &ios);
  if (st != VQ_OK) return st;
  if (T < 0) return fail(VQ_ERR_SHAPE, "T=%d must be >= 0", T);
  if ((int64_t)T * w->num_experts > (1 << 24))
    return fail(VQ_ERR_SHAPE, "T=%d too large (times %d stacked experts)", T, w->num_experts);
  if (T == 0) return VQ_OK;
  if ((int64_t)w->num_experts * ((w->rows + 31) / 32) * ((T + 31) / 32) > (1 << 30))
    return fail(VQ_ERR_SHAPE, "%s: T=%d x %d x %d rows makes too many tiles", name, T, w->num_experts, w->rows);
  st = check_xy(x, y, "y");
  if (st != VQ_OK) return st;
  if (!gemv || T > gemv_token_limit(v, ios))  // above the crossover the MFMA kernel is faster
    return hip_status(vqmi::launch_gemm(v, ios, x, T, y, (hipStream_t)stream),
                      gemv ? "vq_gemv (MFMA path) launch" : "vq_gemm launch");
  return hip_status(vqmi::launch_gemv(v, ios, x, T, y, nullptr, 0, 0, (hipStream_t)stream), "vq_gemv launch");
}

vq_status vq_gemv(const vq_tensor* w, const uint16_t* x, int32_t T, float* y, void* stream) {
  return dense_call(w, nullptr, x, T, y, stream, true);
}

vq_status vq_gemm(const vq_tensor* w, const uint16_t* x, int32_t T, float* y, void* stream) {
  return dense_call(w, nullptr, x, T, y, stream, false);
}

vq_status vq_gemv_ex(const vq_tensor* w, const vq_io* io, const void* x, int32_t T, void* y, void* stream) {
  return dense_call(w, io, x, T, y, stream, true);
}

vq_status vq_gemm_ex(const vq_tensor* w, const vq_io* io, const void* x, int32_t T, void* y, void* stream) {
  return dense_call(w, io, x, T, y, stream, false);
}

vq_status vq_moe_gemv_ex(const vq_tensor* w, const vq_io* io, const void* x, int32_t x_per_slot,
                         const int32_t* expert_ids, int32_t T, int32_t top_k, void* y, void* stream) {
  vqmi::TensorView v;
  vq_status st = check_moe(w, x, x_per_slot, expert_ids, T, top_k, y, &v);
  if (st != VQ_OK) return st;
  vqmi::IoSpec ios;
  st = check_io(io, w, Call::kMoeGemv, &ios);
  if (st != VQ_OK || T == 0) return st;
  if ((int64_t)T * top_k > 65535)
    return fail(VQ_ERR_SHAPE, "vq_moe_gemv: T*top_k=%lld exceeds 65535 pairs; use vq_moe_gemm",
                (long long)T * top_k);
  return hip_status(vqmi::launch_gemv(v, ios, x, T, y, expert_ids, top_k, x_per_slot, (hipStream_t)stream),
                    "vq_moe_gemv launch");
}

vq_status vq_moe_gemv(const vq_tensor* w, const uint16_t* x, int32_t x_per_slot,
                      const int32_t* expert_ids, int32_t T, int32_t top_k, float* y,
                      void* stream) {
  return vq_moe_gemv_ex(w, nullptr, x, x_per_slot, expert_ids, T, top_k, y, stream);
}

size_t vq_moe_workspace_bytes(int32_t T, int32_t top_k, int32_t num_experts) {
  if (T < 0 || top_k < 1 || num_experts < 1 || (int64_t)T * top_k > (1 << 30)) {
    fail(VQ_ERR_SHAPE, "vq_moe_workspace_bytes: bad sizes T=%d top_k=%d num_experts=%d", T, top_k,
         num_experts);
    return 0;
  }
  return vqmi::moe_workspace_bytes(T, top_k, num_experts);
}

vq_status vq_moe_gemm_ex(const vq_tensor* w, const vq_io* io, const void* x, int32_t x_per_slot,
                         const int32_t* expert_ids, int32_t T, int32_t top_k, void* y,
                         void* workspace, size_t workspace_bytes, void* stream) {
  vqmi::TensorView v;
  vq_status st = check_moe(w, x, x_per_slot, expert_ids, T, top_k, y, &v);
  if (st != VQ_OK) return st;
  vqmi::IoSpec ios;
  st = check_io(io, w, Call::kMoeGemm, &ios);
  if (st != VQ_OK || T == 0) return st;
  if (w->num_experts > 1 << 20) return fail(VQ_ERR_SHAPE, "num_experts too large");
  const size_t need = vqmi::moe_workspace_bytes(T, top_k, w->num_experts);
  if (!workspace) return fail(VQ_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(VQ_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(VQ_ERR_ALIGN, "workspace is not 16-byte aligned");
  return hip_status(vqmi::launch_moe_gemm(v, ios, x, x_per_slot, expert_ids, T, top_k, y, workspace,
                                          (hipStream_t)stream),
                    "vq_moe_gemm launch");
}

vq_status vq_moe_gemm(const vq_tensor* w, const uint16_t* x, int32_t x_per_slot,
                      const int32_t* expert_ids, int32_t T, int32_t top_k, float* y,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return vq_moe_gemm_ex(w, nullptr, x, x_per_slot, expert_ids, T, top_k, y, workspace, workspace_bytes,
                        stream);
}

vq_status vq_moe_gemm_no_alloc(const vq_tensor* w, const uint16_t* x, int32_t x_per_slot,
                                const int32_t* expert_ids, int32_t T, int32_t top_k, float* y,
                                void* stream) {
  vqmi::TensorView v;
  vq_status st = check_moe(w, x, x_per_slot, expert_ids, T, top_k, y, &v);
  if (st != VQ_OK || T == 0) return st;
  if (w->num_experts > 1 << 20) return fail(VQ_ERR_SHAPE, "num_experts too large");
  const size_t need = vqmi::moe_workspace_bytes(T, top_k, w->num_experts);
  if (need > vqmi::kStaticScratchBytes)
    return fail(VQ_ERR_WORKSPACE,
                "vq_moe_gemm_no_alloc: T=%d top_k=%d num_experts=%d need %zu bytes of scratch, more than "
                "the %zu bytes of the library's static scratch; use vq_moe_gemm with a workspace",
                T, top_k, w->num_experts, need, vqmi::kStaticScratchBytes);
  void* scratch = nullptr;
  st = hip_status(vqmi::static_scratch(&scratch), "vq_moe_gemm_no_alloc: static scratch address");
  if (st != VQ_OK) return st;
  return hip_status(vqmi::launch_moe_gemm(v, vqmi::IoSpec{}, x, x_per_slot, expert_ids, T, top_k, y, scratch,
                                          (hipStream_t)stream),
                    "vq_moe_gemm_no_alloc launch");
}

// Shape of an encode call (no pointers).
static vq_status check_encode_shape(int32_t rows, int32_t cols, int32_t d, int32_t log2_k, int32_t group,
                                    int32_t n_sample) {
  if ((d != 2 && d != 4 && d != 8) || log2_k < vqmi::kMinBits || log2_k > vqmi::kMaxBits ||
      (group != 64 && group != 128))
    return fail(VQ_ERR_GEOMETRY, "vq_encode: unsupported geometry d=%d log2_k=%d group=%d", d, log2_k, group);
  if (rows < 1 || cols < 1 || cols % group != 0 || (cols / d) % 32 != 0)
    return fail(VQ_ERR_SHAPE, "vq_encode: rows=%d cols=%d: need cols %% group == 0 and (cols/d) %% 32 == 0", rows,
                cols);
  if ((int64_t)rows * cols / d > ((int64_t)1 << 30))
    return fail(VQ_ERR_SHAPE, "vq_encode: more than 2^30 subvectors");
  if (n_sample < 1 || n_sample > (1 << 24))
    return fail(VQ_ERR_SHAPE, "vq_encode: n_sample=%d outside [1, 2^24]", n_sample);
  return VQ_OK;
}

size_t vq_encode_workspace_bytes(int32_t rows, int32_t cols, int32_t d, int32_t log2_k, int32_t n_sample) {
  if (check_encode_shape(rows, cols, d, log2_k, (cols % 64 == 0) ? 64 : 128, n_sample) != VQ_OK) return 0;
  return vqmi::encode_workspace_bytes(rows, cols, d, log2_k, n_sample);
}

vq_status vq_encode(const float* w, int32_t rows, int32_t cols, int32_t d, int32_t log2_k, int32_t group,
                    const int32_t* sample_idx, int32_t n_sample, const double* uniforms, int32_t iters,
                    uint32_t* codes, uint16_t* codebook, uint16_t* scales, double* relerr, void* workspace,
                    size_t workspace_bytes, void* stream) {
  vq_status st = check_encode_shape(rows, cols, d, log2_k, group, n_sample);
  if (st != VQ_OK) return st;
  if (iters < 0) return fail(VQ_ERR_SHAPE, "vq_encode: iters=%d must be >= 0", iters);
  if (!w || !sample_idx || !uniforms || !codes || !codebook || !scales || !relerr)
    return fail(VQ_ERR_NULL, "vq_encode: a required pointer is NULL");
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(codebook, 16) || !aligned(scales, 4) ||
      !aligned(sample_idx, 4) || !aligned(uniforms, 8) || !aligned(relerr, 8))
    return fail(VQ_ERR_ALIGN, "vq_encode: w, codes, codebook need 16-byte alignment; scales, sample_idx 4; "
                              "uniforms, relerr 8");
  const size_t need = vqmi::encode_workspace_bytes(rows, cols, d, log2_k, n_sample);
  if (!workspace) return fail(VQ_ERR_WORKSPACE, "vq_encode: workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(VQ_ERR_WORKSPACE, "vq_encode: workspace has %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(VQ_ERR_ALIGN, "vq_encode: workspace is not 256-byte aligned");
  return hip_status(vqmi::launch_encode(w, rows, cols, d, log2_k, group, sample_idx, n_sample, uniforms, iters, codes,
                                        codebook, scales, relerr, workspace, (hipStream_t)stream),
                    "vq_encode launch");
}

}  // extern "C"
