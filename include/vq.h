/*
 * vq.h -- C ABI of libvqmi.so: fused vector-quantized (VQ) weight matmul on
 * AMD MI355X (gfx950).
 *
 * The operation.  A weight matrix W [rows = out][cols = in] is stored as
 *   - codes: each run of d consecutive weights of a row (along cols) is one
 *     B-bit index (B = log2 K) into a K-entry codebook.  Paper "Data-Free
 *     Vector Quantization Beats Affine Quantization at Matched Bytes Below 5
 *     Bits", Abstract and §1 Notation (geometry dN/KM, log2(K)/d bits/weight).
 *   - codebook: K entries of d fp16 values, one codebook per tensor.  Model
 *     card "Qwen3.5-397B-A17B-VQ-2.4bpw", Methodology (per-tensor fp16
 *     codebook); paper §2.2 (codebook fit on max-abs-scaled subvectors).
 *   - scales: one fp16 scale per (row, group of g weights), g = 64 or 128.
 *     Same card, Methodology (an fp16 scale for each row and 64-weight group); model card
 *     "aquaman164/Qwen3.6-35B-A3B-MLX-VQ-2.4bpw", Recipe (+0.125 bpw: g = 128).
 * and dequantized on the fly:
 *   W[r][c] = fp16( codebook[code(r, c/d)][c % d] * scale[r][c/g] )  (one RNE
 * rounding; the product of two fp16 values is exact in fp32), then
 *   y[t][r] = sum_c W[r][c] * x[t][c]   (fp32 accumulation, fp32 output).
 * The GEMV kernels fold the scale out of each group's inner sum (the sum is
 * formed from exact fp16 x fp16 products in fp32 and multiplied by the scale
 * once per group), which differs from rounding W to fp16 first only by that
 * rounding; vq_dequant and the MFMA GEMM use the rounded W exactly.
 *
 * Code layout (codes packed to their true bit width into uint32 words, each
 * row on its own in blocks of 32 codes: 397B card, Methodology; paper §2.3
 * Packing).  Row r of expert
 * e starts at word (e*rows + r) * Wr, Wr = ceil(cols/d/32) * B.  Code j of a
 * row occupies bits [j*B, (j+1)*B) of the row's little-endian bit stream
 * (least significant bit first); 12-bit codes straddle words.  For B = 8 an
 * array of uint8 codes [rows][cols/d] already is this layout and can be
 * passed as is (397B card, Runtime update: zero-copy packed-8 view).
 *
 * Conventions for every entry point:
 *   - Pointers named as device data point to device memory the caller owns.
 *     The library never allocates device memory; MoE-GEMM scratch comes from
 *     the caller's workspace.
 *   - fp16 values travel as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it without host synchronisation.
 *   - All arguments are validated on the host before anything is enqueued.
 *     On error nothing is enqueued, outputs are untouched, a status is
 *     returned and vq_last_error() describes it.  No C++ exception crosses
 *     the ABI.  Launch failures return VQ_ERR_HIP with HIP's error text.
 *   - Values inside device buffers (codes, expert ids) cannot be checked on
 *     the host.  Every code is in range by construction (B bits).  An expert
 *     id outside [0, num_experts) means "skip": that slot's output row is
 *     written as zeros.
 *   - Calls on one stream are ordered; the library keeps no state between
 *     calls apart from the thread-local error text.
 */
#ifndef VQMI_VQ_H
#define VQMI_VQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VQ_OK = 0,
  VQ_ERR_NULL = 1,      /* a required pointer is NULL                          */
  VQ_ERR_GEOMETRY = 2,  /* (d, log2_k, group) not supported                    */
  VQ_ERR_SHAPE = 3,     /* sizes inconsistent (see each check below)           */
  VQ_ERR_ALIGN = 4,     /* a buffer is not aligned as required                 */
  VQ_ERR_WORKSPACE = 5, /* MoE-GEMM workspace missing or too small             */
  VQ_ERR_HIP = 6        /* a HIP runtime call or kernel launch failed          */
} vq_status;

/*
 * One VQ tensor (dense: num_experts = 1; stacked MoE experts: num_experts = E,
 * one tensor per (layer, projection) holding all experts -- paper, Appendix A,
 * on expert modules).
 *
 * Supported geometry: d in {2, 4, 8}, log2_k in {8, 12}, group in {64, 128}.
 * Shape rules (else VQ_ERR_SHAPE): rows >= 1; cols >= 1; cols % group == 0;
 * group % d == 0; (cols / d) % 32 == 0 (rows hold whole 32-code blocks, so
 * no row needs padding); num_experts >= 1; codebook_per_expert in {0, 1};
 * codebook_elems == E_cb * K * d with E_cb = num_experts if
 * codebook_per_expert else 1.  A codebook sliced across devices or views has
 * the wrong length and is refused rather than read out of bounds (model card
 * "Qwen3.8-27B-VQ-4.5bpw", Multi-machine note: codebooks must be replicated,
 * never sliced, and a sliced one must fail loudly).
 * Alignment (else VQ_ERR_ALIGN): codes 16 bytes; codebook 16 bytes; scales 4
 * bytes.  Size limit (else VQ_ERR_SHAPE): one expert's codes and its scales
 * each fit in 2 GiB - 1 bytes (the kernels address them with 32-bit offsets).
 */
typedef struct vq_tensor {
  const uint32_t *codes;    /* device [E][rows][Wr] packed codes                 */
  const uint16_t *codebook; /* device [E_cb][K][d] fp16 bits, entry-major        */
  const uint16_t *scales;   /* device [E][rows][cols/group] fp16 bits            */
  int32_t rows;             /* output features per expert                        */
  int32_t cols;             /* input features                                    */
  int32_t d;                /* subvector length: 2, 4 or 8                       */
  int32_t log2_k;           /* bits per code B: 8 or 12 (K = 256 or 4096)        */
  int32_t group;            /* weights per scale along a row: 64 or 128          */
  int32_t num_experts;      /* E; 1 for a dense tensor                           */
  int32_t codebook_per_expert; /* 0: one codebook for the tensor; 1: one per expert */
  int64_t codebook_elems;   /* number of fp16 values behind `codebook`           */
} vq_tensor;

/* uint32 words per row of packed codes: ceil(cols/d/32) * log2_k.  Returns -1
 * for a non-positive cols or an unsupported d / log2_k. */
int32_t vq_words_per_row(int32_t cols, int32_t d, int32_t log2_k);

/*
 * Dequantize expert `expert` of `w` to fp16: w_out[r][c] = W[r][c], exactly as
 * defined above (bit-exact).  Used to check the unpack/gather/scale step on
 * its own (397B card and paper §3.4: kernels are accepted on bit-identity
 * with a reference path).  w_out: device [rows][cols] uint16, 16-byte aligned.
 * expert outside [0, num_experts) -> VQ_ERR_SHAPE.
 */
vq_status vq_dequant(const vq_tensor *w, int32_t expert, uint16_t *w_out, void *stream);

/*
 * Decode-shaped product y = x W^T for a dense tensor (num_experts == 1):
 *   x: device [T][cols] fp16 bits, 16-byte aligned;
 *   y: device [T][rows] fp32, 16-byte aligned.
 * T >= 0 (T == 0 enqueues nothing).  Any T is accepted.  The streaming
 * kernel reads every code once per token, the fast path for T = 1 (the fused
 * decode-and-matmul of paper §3.4); above a token count measured per shape
 * (1 for d = 2/4 matrices, 4 for d = 8, 6 for matrices of at most 16M
 * weights) vq_gemv runs the MFMA kernel of vq_gemm instead, with the same
 * result contract.
 */
vq_status vq_gemv(const vq_tensor *w, const uint16_t *x, int32_t T, float *y, void *stream);

/*
 * Prefill-shaped product, same arguments and result as vq_gemv: dequantized
 * weight tiles feed fp16 MFMA instructions with fp32 accumulation.  Any T is
 * accepted; it is the fast path for large T (paper §2.5: scoring runs a
 * prefill-shaped path; §3.4 prefill).  When the output tiles do not fill
 * whole rounds of the GPU's compute units, the tiles of the last, partial
 * round are split along the columns and their partial sums added atomically
 * into y (zeroed first on the same stream): those outputs may differ in the
 * last bits from run to run (fp32 addition order), within the stated
 * tolerance; all others are deterministic.
 */
vq_status vq_gemm(const vq_tensor *w, const uint16_t *x, int32_t T, float *y, void *stream);

/*
 * Routed-expert (top-k MoE) product, decode-shaped: for every token t and
 * slot s, with e = expert_ids[t][s],
 *   y[t][s][:] = W_e x_row  if 0 <= e < num_experts, else zeros,
 * where x_row = x[t] (x_per_slot == 0: gate/up projections, x is [T][cols])
 * or x[t][s] (x_per_slot == 1: down projection, x is [T][top_k][cols]).
 * No router-weight multiply and no combine over slots.  Duplicate ids in a
 * token are computed independently.  (aquaman164 card, Run: fused decode
 * kernels for all expert tiers; Experimental MTP note: decode cost is the
 * routed experts' bytes.)
 *   expert_ids: device [T][top_k] int32, 4-byte aligned;
 *   y: device [T][top_k][rows] fp32, 16-byte aligned;  T >= 0, top_k >= 1,
 *   T * top_k <= 65535 (larger batches belong to vq_moe_gemm), x at most
 *   2 GiB - 1 bytes.
 * Dense projections that share their input (an MLP's gate and up) can be
 * stored as an expert stack (codebook_per_expert = 1 keeps each tensor's own
 * codebook) and run by this call in one launch, with expert_ids {0, 1, ...}
 * in every token: the same results as one vq_gemv per tensor, bit for bit,
 * at one launch's fixed cost.  Routed gate and up projections likewise: with
 * gate_e and up_e stored as experts 2e and 2e + 1 of one stack, expert_ids
 * (2e, 2e + 1) per routed slot and top_k doubled give both outputs of every
 * slot in one launch, bit for bit those of the two separate calls.
 */
vq_status vq_moe_gemv(const vq_tensor *w, const uint16_t *x, int32_t x_per_slot,
                      const int32_t *expert_ids, int32_t T, int32_t top_k, float *y,
                      void *stream);

/* Bytes of workspace vq_moe_gemm needs for these sizes (0 if T*top_k == 0);
 * returns 0 and sets the error text for negative or overflowing sizes. */
size_t vq_moe_workspace_bytes(int32_t T, int32_t top_k, int32_t num_experts);

/*
 * Routed-expert product, prefill-shaped: same arguments and result as
 * vq_moe_gemv.  On the device, the (token, slot) pairs are counted, scanned
 * and scattered by expert, a grouped MFMA GEMM runs over the flat list of
 * (expert, token tile) work items with gathered x rows, and results are
 * written straight to y[t][s].  No host synchronisation.
 *   workspace: device, >= vq_moe_workspace_bytes(T, top_k, num_experts)
 *   bytes, 16-byte aligned, owned by the caller; contents on entry are
 *   ignored and on return are undefined.  Concurrent calls need separate
 *   workspaces.
 * The stacked gate/up layouts described for vq_moe_gemv apply here too
 * (workspace sized for the doubled top_k and expert count): each output row
 * depends only on its expert and x row, so the results are bit for bit those
 * of separate calls.
 */
vq_status vq_moe_gemm(const vq_tensor *w, const uint16_t *x, int32_t x_per_slot,
                      const int32_t *expert_ids, int32_t T, int32_t top_k, float *y,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Text for the last non-OK status returned on this thread ("" if none). */
const char *vq_last_error(void);

/* Name of a status code ("VQ_OK", "VQ_ERR_SHAPE", ...). */
const char *vq_status_name(vq_status s);

#ifdef __cplusplus
}
#endif

#endif /* VQMI_VQ_H */
