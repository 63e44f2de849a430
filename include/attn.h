/*
 * attn.h -- C ABI of libattn: fused scaled-dot-product attention forward for
 * AMD Instinct MI355X (gfx950), with the additive biases and masks of vision
 * transformers.
 *
 *   O = softmax(scale * Q K^T + bias + mask) V,   scale = 1/sqrt(d)
 *
 * The operation: queries and keys, through a softmax, give the attention map
 * whose values weight V; multi-head attention repeats it per head; diffusion
 * models use both self- and cross-attention ("Training and inference
 * acceleration for large vision models", Swin Transformer talk, section 1).
 * The scaled form and its 1/sqrt(d) default are PyTorch's
 * scaled_dot_product_attention ("Accelerated Diffusers with PyTorch 2.0",
 * section "Accelerating transformer blocks").  The biases:
 *   - TABLE: Swin's relative-position bias table (Swin talk, section 1);
 *   - RELPOS: SAM's decomposed relative position, per-query coordinates
 *     indexing Rh/Rw ("Accelerating Generative AI with PyTorch: Segment
 *     Anything, Fast", section "Bfloat16 half precision");
 *   - ADDITIVE: a dense additive tensor.
 * The masks: Swin's shifted-window region mask (Swin talk, section 1) or a
 * dense additive tensor.  Window partition, cyclic shift and their reverses
 * are pure index mappings (Swin talk, section 2) and are folded into the
 * kernel's addressing by ATTN_LAYOUT_IMAGE.
 *
 * Conventions
 *  - All tensor pointers are DEVICE pointers owned by the caller; they must
 *    stay valid until the work queued on `stream` has finished.  The library
 *    allocates nothing, keeps no pointer after returning, holds no mutable
 *    global state (apart from the per-device address of attn_bwd_noalloc's
 *    fixed array, taken once), and is safe to call from several host
 *    threads.
 *  - attn_fwd never synchronises the device and never copies host memory to
 *    the device: every index computation (bias gathers, window and shift
 *    maps, region labels) happens inside the kernel from by-value integers.
 *    (The pages trace a hidden host sync to indexing with host tensors, SAM
 *    blog, sections "Baseline" and "Bfloat16"; this ABI has none.)
 *  - Descriptors themselves are HOST structs read during the call only.
 *  - Results are deterministic: identical inputs give bitwise-identical
 *    outputs (no atomics, fixed reduction order).
 *  - Errors are returned as status codes; nothing is thrown or aborted
 *    across the ABI.  NaN/Inf in the inputs are not checked; they propagate
 *    to the affected output rows.  A row whose logits are all -inf (only
 *    possible through an ADDITIVE mask/bias) produces NaN, as the plain
 *    definition does.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_API __attribute__((visibility("default")))

/* Status codes. */
enum {
  ATTN_OK = 0,
  ATTN_E_NULL = 1,        /* a required pointer is NULL                        */
  ATTN_E_SHAPE = 2,       /* inconsistent B/H/N/d, grid or window geometry     */
  ATTN_E_LAYOUT = 3,      /* bad strides or alignment                          */
  ATTN_E_UNSUPPORTED = 4, /* head_dim, dtype or size outside what is built     */
  ATTN_E_ALIAS = 5,       /* out overlaps q, k or v                            */
  ATTN_E_LAUNCH = 6,      /* the HIP launch reported an error                  */
  ATTN_E_INVALID = 7      /* an enum value or field is out of range            */
};

/* Element type of q, k, v, out, the bias tables and dense bias/mask tensors. */
typedef enum { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 } attn_dtype_t;

/* Token layout of a tensor.
 *  BATCHED: dims = {B_eff, H, N, d}; windows are extra batch items.
 *  IMAGE:   dims = {B_img, H, img_h*img_w, d}, tokens in image row-major
 *           order.  The kernel pads the image to whole windows (see
 *           attn_window_t), partitions it into win_h x win_w windows (after
 *           a cyclic shift by (shift_h, shift_w) when they are non-zero) and
 *           writes `out` back in image order, i.e. reverse partition, reverse
 *           shift and crop.  The window geometry is taken from
 *           mask_desc->win.  Batch item b_eff = img * nW + window, windows
 *           row-major.  q, k, v and out must all use IMAGE together; every
 *           element offset inside one (image, head) slice must be below 2^29
 *           (E_UNSUPPORTED otherwise).                                       */
typedef enum { ATTN_LAYOUT_BATCHED = 0, ATTN_LAYOUT_IMAGE = 1 } attn_layout_t;

/* A strided 4-D tensor [B, H, N, d]; the d stride is 1.
 * strides[] are in ELEMENTS for the B, H and N axes.  `data` must be 16-byte
 * aligned and every stride a multiple of 16 bytes (8 elements for f16/bf16,
 * 4 for f32): the kernels move rows in 16-byte pieces (ATTN_E_LAYOUT).
 * Exception: q, k and v given as 8-bit codes (attn_options_t.qkv_format =
 * ATTN_QKV_E4M3) need 8-byte alignment of `data` and strides that are
 * multiples of 8 elements; they are moved in 8-byte pieces.                 */
typedef struct {
  void* data;
  int64_t dims[4];
  int64_t strides[3];
  int32_t layout; /* attn_layout_t */
} attn_tensor_t;

typedef enum {
  ATTN_BIAS_NONE = 0,
  ATTN_BIAS_TABLE = 1,    /* bias[i,j] = table[(qh-kh+gh-1)*(2gw-1) + (qw-kw+gw-1), head] */
  ATTN_BIAS_RELPOS = 2,   /* bias[i,j] = q_i.Rh[qh-kh+gh-1] + q_i.Rw[qw-kw+gw-1] (equal
                             query and key grids; see kgrid_h below otherwise)         */
  ATTN_BIAS_ADDITIVE = 3  /* bias[i,j] = add[b % add_batch, i, j]                          */
} attn_bias_kind_t;

/* Bias descriptor.
 *  grid_h, grid_w: token grid of one batch item (window or image); required
 *    for TABLE and RELPOS, where Nq = Nk = grid_h * grid_w and token t sits
 *    at (t / grid_w, t % grid_w).
 *  kgrid_h, kgrid_w: RELPOS only, BATCHED layout only: the key grid when it
 *    differs from the query grid (both 0: the key grid is grid_h x grid_w;
 *    must be 0 for the other kinds).  Then Nq = grid_h*grid_w,
 *    Nk = kgrid_h*kgrid_w, and per axis (n query, m key positions) the table
 *    row of query coordinate a and key coordinate c is
 *    floor(a*max(m/n,1) - c*max(n/m,1) + (m-1)*max(n/m,1)) in exact
 *    arithmetic: the shorter axis is stretched onto the longer one, as the
 *    coordinate scalers of SAM's image encoder do ("Accelerating Generative
 *    AI with PyTorch: Segment Anything, Fast", section "Bfloat16 half
 *    precision").  Rh and Rw then need 2*max(grid_h,kgrid_h)-1 and
 *    2*max(grid_w,kgrid_w)-1 rows.
 *  rh_rows, rw_rows: RELPOS only: the rows Rh and Rw actually hold (0: the
 *    rows needed, above).  A table of another length (1 to 1023 rows) is
 *    resized in the kernel to the needed length by linear interpolation
 *    along the offset axis with both end rows kept: needed row r reads the
 *    stored table at position r*(L-1)/(M-1) for L stored and M needed rows
 *    (rel_pos_resized of the same SAM write-ups, which name the resize
 *    without its rule).  Must be 0 for the other kinds.
 *  table: [(2gh-1)(2gw-1), H] contiguous, element [r, head] at r*H + head.
 *  rh: [rh_rows, d], rw: [rw_rows, d] contiguous, by default [2gh-1, d] and
 *    [2gw-1, d] (longer with a key grid, see above), shared by all heads;
 *    they are dotted with the raw (unscaled) query row; the bias is not
 *    scaled.  Both must be 16-byte aligned.
 *  add: [add_batch, Nq, Nk] with element strides add_strides[0..1] for the
 *    first two axes, last stride 1; batch item b uses add[b % add_batch].
 *  All bias data uses the call's dtype.                                     */
typedef struct {
  int32_t kind; /* attn_bias_kind_t */
  int32_t grid_h, grid_w;
  const void* table;
  const void* rh;
  const void* rw;
  const void* add;
  int64_t add_batch;
  int64_t add_strides[2];
  int32_t kgrid_h, kgrid_w;
  int32_t rh_rows, rw_rows;
} attn_bias_desc_t;

typedef enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_ADDITIVE = 1,      /* mask[i,j] = add[b % n_win, i, j]                       */
  ATTN_MASK_SHIFT_REGIONS = 2  /* mask[i,j] = value if region(i) != region(j), else 0     */
} attn_mask_kind_t;

/* Window geometry (Swin, SAM).  img_h, img_w: token image; win_h, win_w:
 * window; shift_h, shift_w: cyclic shift, 0 <= shift < win.
 * When the image is not a whole number of windows it is zero-padded at the
 * bottom and right to the padded grid PH = ceil(img_h/win_h)*win_h,
 * PW = ceil(img_w/win_w)*win_w (SAM's 64x64 token grid in 14x14 windows is
 * padded to 70x70: the windowed-encoder workload, and zero padding of the
 * encoder input for static shapes, "Accelerating Generative AI with PyTorch:
 * Segment Anything, Fast", section "Torch.compile").  Padded tokens have
 * q = k = v = 0 and take part in the attention like any other token (no key
 * masking); their outputs are not written.  The shift and the regions are
 * taken on the padded grid: shifted pixel (Y, X) holds padded pixel
 * ((Y+shift_h) mod PH, (X+shift_w) mod PW), and its region is 3*ry + rx with
 * ry = 0 for Y < PH-win_h, 1 for Y < PH-shift_h, 2 otherwise (same for X).
 * Used by SHIFT_REGIONS and by ATTN_LAYOUT_IMAGE.                            */
typedef struct {
  int32_t img_h, img_w, win_h, win_w, shift_h, shift_w;
} attn_window_t;

/* Mask descriptor.
 *  add: [n_win, Nq, Nk], element strides add_strides[0..1], last stride 1,
 *    batch item b uses add[b % n_win].
 *  win: window geometry (SHIFT_REGIONS and IMAGE layout).  In BATCHED layout
 *    SHIFT_REGIONS labels batch item b as window b % nW of an image, where
 *    nW = (PH/win_h)*(PW/win_w) windows of the padded grid.
 *  value: the additive value for pairs from different regions (Swin uses
 *    -100).                                                                  */
typedef struct {
  int32_t kind; /* attn_mask_kind_t */
  const void* add;
  int64_t n_win;
  int64_t add_strides[2];
  attn_window_t win;
  float value;
} attn_mask_desc_t;

/* attn_fwd: queue O = softmax(QK^T/sqrt(d) + bias + mask) V on `stream`.
 *
 *  q: [B, H, Nq, d]; k, v: [B, H, Nk, d]; out: [B, H, Nq, d] (written).
 *  bias_desc, mask_desc: may be NULL, meaning NONE.
 *  dtype: element type of every tensor and table.
 *  stream: a hipStream_t (NULL = the default stream), passed as void*.
 *
 *  Supported: d in {32, 40, 64, 80} for F16/BF16; d <= 128, d % 4 == 0 for
 *  F32.  Nq, Nk >= 1.  Within one (batch item, head) slice every element
 *  offset, (N-1)*N-stride + d, must be below 2^31 (else
 *  ATTN_E_UNSUPPORTED).  TABLE/RELPOS/SHIFT_REGIONS need Nq == Nk ==
 *  grid_h*grid_w (SHIFT_REGIONS: == win_h*win_w).  A call whose kernel would
 *  need more than the 160 KiB of LDS of one CU for its tiles and per-query
 *  bias tables (RELPOS on large grids other than 64 wide, key grids with
 *  long axes) returns ATTN_E_UNSUPPORTED; so does a grid of more than
 *  2^31-1 workgroups.
 *  Returns ATTN_OK after queueing the kernel, or an error code (nothing is
 *  queued on error).  Asynchronous: kernel faults surface at the caller's
 *  next synchronisation.                                                     */
ATTN_API int attn_fwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
             const attn_bias_desc_t* bias_desc, const attn_mask_desc_t* mask_desc,
             const attn_tensor_t* out, int32_t dtype, void* stream);

/* attn_check: the validation attn_fwd performs, without touching the GPU.
 * Same arguments minus the stream; returns the status attn_fwd returns for
 * the same arguments, short of a launch failure (ATTN_OK if attn_fwd would
 * queue the kernel), including ATTN_E_UNSUPPORTED for calls whose tiles
 * and tables do not fit in LDS.                                              */
ATTN_API int attn_check(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
               const attn_bias_desc_t* bias_desc, const attn_mask_desc_t* mask_desc,
               const attn_tensor_t* out, int32_t dtype);

/* Storage format of q, k and v (attn_options_t.qkv_format).
 *  DTYPE: elements of the call's dtype, like out and the tables.
 *  E4M3:  one byte per element, the E4M3 format of the OCP 8-bit floating
 *         point specification (sign, 4-bit exponent with bias 7, 3-bit
 *         mantissa, subnormals, no infinities, S.1111.111 = NaN), each
 *         tensor with one scale: the value of a code is code * scale.  The
 *         attention is computed on those values exactly as on dtype inputs
 *         (dtype must be F16 or BF16, the matrix-core compute and output
 *         type).  The low-precision reading follows the pages' use of
 *         quantized products whose quantization and dequantization are fused
 *         into the neighbouring operators ("Training and inference
 *         acceleration for large vision models", section 3; "Accelerating
 *         Generative AI with PyTorch: Segment Anything, Fast", introduction,
 *         GPU quantization): here the dequantization is fused into the
 *         attention's loads.                                                 */
typedef enum { ATTN_QKV_DTYPE = 0, ATTN_QKV_E4M3 = 1 } attn_qkv_format_t;

/* Options of attn_fwd_opt / attn_check_opt.
 *  window_heads: for windows of at most 64 tokens in half precision (TABLE
 *    or no bias, SHIFT_REGIONS or no mask), how many heads of one window
 *    share a workgroup.  0: the library's choice (currently one head per
 *    workgroup, the fastest form measured on MI355X for Swin windows);
 *    1: one head per workgroup; 2, 3 or 4: that many heads of a window per
 *    workgroup, which then computes the window's index data (key offsets,
 *    region labels, table staging) once for all of them -- the short-
 *    sequence packing of windows into workgroups.  A value that does not
 *    divide H, a value above 4, or a call outside the short-sequence path
 *    with a value above 1 returns ATTN_E_UNSUPPORTED (negative: E_INVALID).
 *  qkv_format: attn_qkv_format_t of q, k and v (0: the call's dtype).  With
 *    ATTN_QKV_E4M3, q_descale, k_descale and v_descale are the three
 *    tensors' scales (finite and > 0, else ATTN_E_INVALID); dtype F32 and
 *    the RELPOS bias return ATTN_E_UNSUPPORTED, and so does window_heads
 *    above 1.  Tables, dense bias/mask tensors and out keep the dtype.
 *  lse: NULL, or device fp32 memory (4-byte aligned, overlapping no input
 *    or output) that receives each query row's log-sum-exp of its logits,
 *    L_i = log sum_j exp(scale*q_i.k_j + bias_ij + mask_ij) (natural log):
 *    [B, H, Nq] contiguous, in the IMAGE layout [images, H, img_h*img_w]
 *    in image order (padding tokens have no entry).  attn_bwd_opt takes it
 *    back.  Half precision only (also with 8-bit inputs) and window_heads
 *    at most 1, else ATTN_E_UNSUPPORTED.
 *  Zero-initialise the struct: fields added later keep 0 as "library's
 *  choice".                                                                  */
typedef struct {
  int32_t window_heads;
  int32_t qkv_format;
  float q_descale, k_descale, v_descale;
  int32_t reserved;
  float* lse;
} attn_options_t;

/* attn_fwd_opt / attn_check_opt: attn_fwd / attn_check with options (NULL:
 * all defaults, identical to attn_fwd / attn_check).  The packing of Swin
 * windows into workgroups is described for the method's short sequences
 * ("Training and inference acceleration for large vision models", section 1:
 * attention inside each window).                                             */
ATTN_API int attn_fwd_opt(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                 const attn_bias_desc_t* bias_desc, const attn_mask_desc_t* mask_desc,
                 const attn_tensor_t* out, int32_t dtype, const attn_options_t* options,
                 void* stream);
ATTN_API int attn_check_opt(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                   const attn_bias_desc_t* bias_desc, const attn_mask_desc_t* mask_desc,
                   const attn_tensor_t* out, int32_t dtype, const attn_options_t* options);

/* Backward pass: gradients of L = sum(dout * O) for the forward
 * O = softmax(scale*QK^T + bias + mask) V ("Training and inference
 * acceleration for large vision models", section 2: Swin is trained with a
 * fused window op that has a forward and a backward).
 *
 *  q, k, v, bias_desc, mask_desc, dtype: as in attn_fwd.  dout: the output
 *  gradient, laid out like `out` of attn_fwd.  dq, dk, dv: written, shaped and
 *  laid out like q, k, v (own strides allowed); they must overlap no input and
 *  no other gradient.  dtable (4-byte aligned device fp32, overwritten; may
 *  be NULL for the other bias kinds): TABLE bias: [(2gh-1)(2gw-1), H],
 *  element [r, head] at r*H + head, the table gradient summed over all
 *  batch items and windows.  RELPOS: [(2gh-1) + (2gw-1), d], the gradient
 *  of Rh (its 2gh-1 rows first) and then of Rw, summed over all batch items
 *  and heads -- through the decomposed bias rel_h[i][kh] + rel_w[i][kw]
 *  ("Accelerating Generative AI with PyTorch: Segment Anything, Fast",
 *  section "Bfloat16").  The mask and an ADDITIVE bias receive no gradient.
 *  workspace: device memory of at least the bytes attn_bwd_workspace_size
 *    reports, 16-byte aligned, owned by the caller (NULL allowed when that is
 *    0); its contents before and after the call are unspecified.  Window
 *    units: B_eff * H * table rows * 4 bytes with a TABLE bias (the
 *    per-window partial table gradients, summed over windows in a fixed
 *    order by a second kernel), else 0.  Longer sequences: 2 * B * H * Nq * 4
 *    bytes (each query row's log-sum-exp and sum_j P_ij dP_ij); with RELPOS
 *    also each query's rel_h / rel_w rows (B * H * Nq * (gh + gw) floats;
 *    B * H * Nq * 32 floats when gh + gw <= 32 and Nk <= 256, a row then
 *    being 32 columns in the element type, high and low parts) and one
 *    partial [dRh; dRw] per 64 query rows (B * H * ceil(Nq / 64)
 *    slots of ((2gh-1) + (2gw-1)) * d floats, at least (gh + 64) * 64 when
 *    gw = 64), summed in a fixed order; these two regions start on multiples
 *    of 4 floats.  Bitwise-deterministic, no atomics.
 *
 *  Built: half precision (F16/BF16).  Units of at most 64 queries and keys
 *  (the window path: Swin windows in either layout, with shift and padding
 *  folded in) with bias NONE, TABLE or ADDITIVE and any mask; longer
 *  sequences in the batched layout without a mask and with no bias (SD-
 *  style self- and cross-attention) or the RELPOS bias on equal query and
 *  key grids with tables of 2g-1 rows (SAM's windowed and global layers;
 *  grid width 64, or gh + gw <= 84, 83 at d = 80): a row kernel (log-sum-exp, D, dQ and
 *  the relative-position terms) and a column kernel (dK, dV).  Other calls
 *  (fp32, key grids or resized tables, other biases or masks on long
 *  sequences, the image layout beyond 64 tokens) return
 *  ATTN_E_UNSUPPORTED.  Asynchronous on `stream`.                             */
ATTN_API int attn_bwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
             const attn_tensor_t* dout, const attn_bias_desc_t* bias_desc,
             const attn_mask_desc_t* mask_desc, const attn_tensor_t* dq, const attn_tensor_t* dk,
             const attn_tensor_t* dv, float* dtable, int32_t dtype, void* workspace,
             size_t workspace_bytes, void* stream);

/* Options of attn_bwd_opt: the forward's results for the same call.
 *  out: the forward output O (laid out like dout) and lse: its per-row
 *    log-sum-exp (attn_options_t.lse of the forward).  Given together
 *    (both non-NULL), the tiled path takes each row's normaliser from lse
 *    and D_i = sum_j P_ij dP_ij from dO_i . O_i instead of a pass over the
 *    keys of its own (the identity sum_j P_ij (dO_i . v_j) = dO_i . O_i);
 *    the window path, which recomputes P exactly, ignores them.  Both NULL:
 *    identical to attn_bwd.  One of them NULL: ATTN_E_NULL.
 *  Zero-initialise the struct.                                               */
typedef struct {
  const attn_tensor_t* out;
  const float* lse;
  int32_t reserved[4];
} attn_bwd_options_t;

/* attn_bwd_opt: attn_bwd with options (NULL: identical to attn_bwd).        */
ATTN_API int attn_bwd_opt(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                 const attn_tensor_t* dout, const attn_bias_desc_t* bias_desc,
                 const attn_mask_desc_t* mask_desc, const attn_tensor_t* dq, const attn_tensor_t* dk,
                 const attn_tensor_t* dv, float* dtable, int32_t dtype,
                 const attn_bwd_options_t* options, void* workspace, size_t workspace_bytes,
                 void* stream);

/* attn_bwd_check: the validation of attn_bwd without touching the GPU (the
 * status attn_bwd returns, short of a launch failure).                       */
ATTN_API int attn_bwd_check(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                   const attn_tensor_t* dout, const attn_bias_desc_t* bias_desc,
                   const attn_mask_desc_t* mask_desc, const attn_tensor_t* dq,
                   const attn_tensor_t* dk, const attn_tensor_t* dv, float* dtable,
                   int32_t dtype, void* workspace, size_t workspace_bytes);

/* attn_bwd_workspace_size: *bytes = the workspace attn_bwd needs for these
 * arguments (validated as the forward call with dout as its output).         */
ATTN_API int attn_bwd_workspace_size(const attn_tensor_t* q, const attn_tensor_t* k,
                            const attn_tensor_t* v, const attn_tensor_t* dout,
                            const attn_bias_desc_t* bias_desc, const attn_mask_desc_t* mask_desc,
                            int32_t dtype, size_t* bytes);

/* attn_bwd_noalloc: attn_bwd without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The per-window table
 * gradients (or the rows' statistics) go to a fixed 16 MiB device array of
 * the library (one per device, held until the process ends) instead: a call
 * whose workspace
 * would exceed it (attn_bwd_workspace_size > 16 MiB, e.g. more than 8272
 * windows of 7x7 tokens with 3 heads) returns ATTN_E_UNSUPPORTED.  No
 * allocation of any kind.  Every call on a device shares that device's
 * array, so calls that overlap on one device (other streams or host
 * threads) race on it; sequential calls on one stream are safe.  Otherwise
 * identical to attn_bwd (same validation, kernels and results).             */
ATTN_API int attn_bwd_noalloc(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                     const attn_tensor_t* dout, const attn_bias_desc_t* bias_desc,
                     const attn_mask_desc_t* mask_desc, const attn_tensor_t* dq,
                     const attn_tensor_t* dk, const attn_tensor_t* dv, float* dtable,
                     int32_t dtype, void* stream);

/* attn_strerror: static text for a status code (never NULL).                */
ATTN_API const char* attn_strerror(int status);

/* attn_version: library ABI version, (major << 16) | minor (1.2 added
 * attn_fwd_opt, attn_check_opt and the rh_rows, rw_rows fields of
 * attn_bias_desc_t, which grew from 80 to 88 bytes; 1.3 the backward:
 * attn_bwd, attn_bwd_check, attn_bwd_workspace_size; 1.4 8-bit q, k, v:
 * qkv_format and the three scales in attn_options_t, whose size is
 * unchanged; 1.5 the lse output of attn_options_t and attn_bwd_opt).        */
ATTN_API int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
