/*
 * mq.h: C ABI of the Matryoshka-nested integer matmul library (libmq.so),
 * gfx950 (MI355X) only.
 *
 * The method ("Matryoshka Quantization" explainer, §3.4): a model is stored
 * once as unsigned 8-bit codes q with an fp32 scale alpha and zero point z per
 * weight vector (min-max quantizer, Eq. 1).  At serve time the codes are
 * sliced to their r most significant bits with rounding and clamping,
 *   S(q, r) = clamp(round(q / 2^(8-r)), 0, 2^r - 1) * 2^(8-r)       (Eq. 6),
 * dequantized as (S(q, r) - z) * alpha (the sliced value is used as if it
 * were an int8 value, "The Bit-Slicing Operator"), and multiplied by bf16
 * activations with fp32 accumulation.  Different layers may use different r
 * over the one stored model ("Mix'n'Match").
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc or torch CUDA
 *    tensors), owned by the caller, which keeps them alive until the work
 *    enqueued on `stream` has finished.  Inputs and outputs must not overlap.
 *  - A weight matrix has logical shape [N, K] (N outputs, K inputs), stored
 *    row-major with K contiguous: the transpose of the pages' W in X W.
 *  - `group` is the length of the weight vector that owns one (alpha, z):
 *    group == K (per output channel) or group == 128 (128 consecutive inputs
 *    of a row).  alpha and zero are fp32 [N, K / group] row-major.
 *  - Activations are bf16 bit patterns (uint16_t) [M, K] row-major; outputs
 *    are fp32 [M, N] row-major.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    and the call returns without synchronizing.
 *  - Every argument is validated before anything is enqueued: on an error
 *    nothing is enqueued and no output is touched.  A failed launch returns
 *    MQ_ERR_HIP and records the hipError_t (see mq_last_hip_error).  Faults
 *    during execution surface at the caller's next synchronization.
 *  - No entry point allocates device memory.  The library keeps no state
 *    except cached device properties and, once mq_gemm_noalloc has run on a
 *    device, that device's scratch array.  Calls are thread-safe (except
 *    that overlapping mq_gemm_noalloc calls on one device share its scratch).
 */
#ifndef MQ_H
#define MQ_H

#include <stddef.h>
#include <stdint.h>

/* The library is built with hidden visibility; these entry points are the
 * only symbols it exports. */
#if defined(__GNUC__) || defined(__clang__)
#define MQ_API __attribute__((visibility("default")))
#else
#define MQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mq_status {
  MQ_OK = 0,
  MQ_ERR_NULL = 1,      /* a required pointer is NULL                          */
  MQ_ERR_SHAPE = 2,     /* a size is out of range (see each entry point)       */
  MQ_ERR_PRECISION = 3, /* r is not 2, 3, 4, 6 or 8 */
  MQ_ERR_GROUP = 4,     /* group is neither K nor 128                          */
  MQ_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned                    */
  MQ_ERR_WORKSPACE = 6, /* workspace missing or smaller than required          */
  MQ_ERR_DEVICE = 7,    /* the current device is not a gfx950                  */
  MQ_ERR_HIP = 8        /* a HIP runtime call failed                            */
} mq_status;

/* Human-readable name of a status code (static string, never NULL). */
MQ_API const char* mq_status_string(int status);

/* hipError_t value recorded by the last MQ_ERR_HIP returned on this thread
 * (0 if none). */
MQ_API int mq_last_hip_error(void);

/* Library version string, e.g. "mq 0.1 gfx950". */
MQ_API const char* mq_version(void);

/* Bytes of one packed r-bit plane of an [N, K] matrix: N * K * r / 8.
 * Returns 0 for r not in {2, 3, 4, 6, 8} or negative sizes. */
MQ_API size_t mq_packed_bytes(int64_t N, int64_t K, int r);

/*
 * mq_quantize: min-max quantization of fp32 weights to 8-bit codes
 * ("Matryoshka Quantization" explainer, §3.4 "Quantization Primitives", Eq. 1,
 * with c = 8).  For every weight vector v (group consecutive entries of a row):
 *   alpha = fp32((max v - min v) / 255),  z = fp32(-min v / alpha),
 *   q = clamp(floor(v / alpha + z + 1/2), 0, 255),
 * evaluated in IEEE float64 from the stored fp32 alpha and z.  A constant
 * vector gets alpha = 1, z = -min (all codes 0); so does a vector whose range
 * is so small that its fp32 alpha would be 0 or subnormal (below 2^-126), so
 * every alpha written is a normal fp32 number.
 *   w      fp32 [N, K], finite values
 *   codes  uint8 [N, K] (output)
 *   alpha  fp32 [N, K/group] (output), zero fp32 [N, K/group] (output)
 * Sizes: N >= 1, K >= 1, group divides K and group == K or group == 128.
 */
MQ_API mq_status mq_quantize(const float* w, int64_t N, int64_t K, int64_t group,
                      uint8_t* codes, float* alpha, float* zero, void* stream);

/*
 * mq_pack: slice stored codes to r bits and pack them (Eq. 6; the explainer's
 * §2 and "The Bit-Slicing Operator": a lower-precision model is extracted from
 * the one stored int8 model by slicing; r = 3 and 6 are the interpolated
 * precisions of "Mix'n'Match and Interpolative Slicing").  Writes, for every
 * code,
 *   t = min((q + 2^(7-r)) >> (8-r), 2^r - 1)   (r < 8),   t = q   (r = 8),
 * the index with S(q, r) = t * 2^(8-r).
 * Layout (r = 2, 4, 8): each row is cut into little-endian 32-bit words of
 * 32/r consecutive indices; the indices at even positions fill the low 16
 * bits, those at odd positions the high 16 bits, the j-th of a half in bits
 * [j*r, j*r + r) of that half.
 * Layout (r = 3, 6): two planes back to back, each in the layout above: first
 * t >> r_lo for all rows (width r - r_lo), then t & (2^r_lo - 1) for all rows
 * (width r_lo = 1 for r = 3, 2 for r = 6).
 *   codes   uint8 [N, K]
 *   packed  uint8, N*K*r/8 bytes (output), 16-byte aligned
 * Sizes: N >= 1, K >= 64, K % 64 == 0; r in {2, 3, 4, 6, 8}.
 */
MQ_API mq_status mq_pack(const uint8_t* codes, int64_t N, int64_t K, int r, uint8_t* packed,
                  void* stream);

/*
 * mq_gemv: decode-shaped product against an r-bit plane, M <= 8 rows of
 * activations:
 *   y[m, n] = sum_k x[m, k] * (S(q[n, k], r) - z[n, g]) * alpha[n, g],
 *   g = k / group,
 * with the slice read from `packed` (the output of mq_pack for the same r),
 * bf16 x, fp32 accumulation and an fp32 result.  The weight is the sliced
 * code dequantized with the int8 code's own alpha and z: the "Matryoshka
 * Quantization" explainer, §3.4 "The Bit-Slicing Operator" (Eq. 6; a sliced
 * value is used in computation like an int8 value) and "Quantization
 * Primitives" (Eq. 1, dequantization alpha * (q - z)).  At batch 1 the time is
 * set by moving the planes out of HBM (the explainer's §2 "Context").
 * alpha must hold finite normal fp32 numbers (as mq_quantize writes them).
 *   packed  uint8 [N, K*r/8], 16-byte aligned
 *   alpha, zero  fp32 [N, K/group]
 *   x       bf16 bits [M, K], 16-byte aligned
 *   y       fp32 [M, N] (output), 16-byte aligned
 * Sizes: 1 <= M <= 8, N >= 1, K >= 64, K % 64 == 0, K <= 65536;
 * r in {2, 3, 4, 6, 8}.
 */
MQ_API mq_status mq_gemv(const uint8_t* packed, int r, const float* alpha, const float* zero,
                  int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                  float* y, void* stream);

/* One product of a grouped GEMV launch (see mq_gemv_grouped). */
typedef struct mq_gemv_problem {
  const uint8_t* packed; /* uint8 [N, K*r/8]                 */
  const float* alpha;    /* fp32 [N, K/group]                */
  const float* zero;     /* fp32 [N, K/group]                */
  const uint16_t* x;     /* bf16 bits [M, K]                 */
  float* y;              /* fp32 [M, N] (output)             */
  int64_t N, K, group;
} mq_gemv_problem;

/*
 * mq_gemv_grouped: several independent mq_gemv products at the same r and M
 * in one launch (for example the three matrices of a feed-forward block, or
 * the projections that share one input).  Same definitions, constraints and
 * result as calling mq_gemv on each problem; outputs must not overlap.
 * 1 <= count <= 16.
 */
MQ_API mq_status mq_gemv_grouped(const mq_gemv_problem* problems, int count, int r, int64_t M,
                          void* stream);

/*
 * mq_gemv_mixed: as mq_gemv_grouped, but problem i is sliced to its own
 * precision r[i] (2, 3, 4, 6 or 8): several precisions of one stored int8 model
 * served in one launch ("Matryoshka Quantization" explainer, §3.4
 * "Mix'n'Match and Interpolative Slicing": any r, chosen per consumer, from
 * the same codes).  Each result equals mq_gemv on that problem at r[i].
 *   r  host array of `count` precisions, read during the call only
 * Problems with per-channel and group-128 scales may be mixed; they take one
 * launch per granularity.  1 <= count <= 16.
 */
MQ_API mq_status mq_gemv_mixed(const mq_gemv_problem* problems, const int* r, int count, int64_t M,
                        void* stream);

/*
 * mq_gemm: the same product for any number of activation rows M >= 1 (small
 * batches and prefill), on bf16 matrix cores with fp32 accumulation:
 *   y[m, n] = sum_k x[m, k] * (S(q[n, k], r) - z[n, g]) * alpha[n, g]
 * (the explainer's §3.4, Eq. 6 slicing and the Eq. 1 dequantization with the
 * int8 code's alpha and z; group 128 is the per-group granularity of the
 * "Pith review of ROSAQ").  Same definitions and layouts as mq_gemv; M <= 8
 * takes the mq_gemv kernel.  alpha must hold finite normal fp32 numbers whose
 * ratio between consecutive groups of a row is finite (true of every alpha
 * mq_quantize writes for weights below 2^100 in magnitude).
 * Every r in {2, 3, 4, 6, 8} is served at every M (r = 3 and 6 from their
 * high- and low-bit planes).
 *   workspace  device scratch of at least mq_gemm_workspace_bytes(M, N, K, group)
 *              bytes (may be NULL when that is 0), 256-byte aligned: the fp32
 *              partial products of K slices, used where the output tiles alone
 *              leave the chip idle (small batches; larger M with long K or
 *              few output columns, e.g. a 4096-wide down projection)
 * Sizes: M >= 1, N >= 1, K >= 64, K % 64 == 0, K <= 65536.
 */
/* Workspace bytes of mq_gemm.  It takes N as well as M, K and group because
 * the workspace holds one fp32 [M, N] partial product per K slice; 0 when the
 * shape is served without a K split. */
MQ_API size_t mq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group);
MQ_API mq_status mq_gemm(const uint8_t* packed, int r, const float* alpha, const float* zero,
                  int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * mq_gemm_noalloc: mq_gemm for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, result and validation as
 * mq_gemm without the workspace: the K-slice partial products go to a scratch
 * array inside the library, MQ_GEMM_NOALLOC_MAX_BYTES (64 MiB) per device,
 * held from the first call on that device until the process ends.  Returns
 * MQ_ERR_WORKSPACE, enqueuing nothing, when the shape needs more than that
 * (mq_gemm_workspace_bytes(M, N, K, group) > MQ_GEMM_NOALLOC_MAX_BYTES).
 * The call allocates nothing.  Every call on one device shares that device's
 * array: calls that may overlap in time on one device (other streams, other
 * threads) race and must be serialized by the caller.
 */
#define MQ_GEMM_NOALLOC_MAX_BYTES ((size_t)64 << 20)
MQ_API mq_status mq_gemm_noalloc(const uint8_t* packed, int r, const float* alpha, const float* zero,
                          int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                          float* y, void* stream);

/*
 * Extra-Precision MatQuant: the slice without the clamp (the errata Eq. 8 of
 * the explainer's "The Bit-Slicing Operator") has 2^r + 1 levels; the extra
 * one, 256, is reached by the codes q >= 256 - 2^(7-r) (none at r = 8).  The
 * r-bit plane of mq_pack keeps the clamped index; these calls list the codes
 * at the extra level per row and add their missing 2^(8-r) * alpha * x to a
 * product, which gives the extra-precision product ([MQX] §5 "Critical
 * Assessment": such sparse additions need a kernel of their own).
 *
 * mq_overflow_rows: row_ptr int32 [N + 1] (output): row_ptr[0] = 0 and
 *   row_ptr[n + 1] - row_ptr[n] = number of such codes in row n.
 * mq_overflow_cols: col_idx uint16 [row_ptr[N]] (output, 2-byte aligned):
 *   their column k, row by row, increasing within a row (row_ptr as written
 *   by mq_overflow_rows; the caller reads row_ptr[N] to size col_idx).  The
 *   lists cost 16 bits per listed code plus 32 per row.
 * mq_overflow_apply: y[m, n] += 2^(8-r) * sum over row n's listed k of
 *   alpha[n, k/group] * x[m, k], summed in a fixed order (deterministic).
 *   Run after mq_gemv / mq_gemm at the same r on the same y.
 * codes uint8 [N, K] 16-byte aligned; x bf16 bits [M, K]; y fp32 [M, N].
 * Sizes: N >= 1, K >= 64, K % 64 == 0, K <= 65536, N * K < 2^31; M >= 1.
 */
MQ_API mq_status mq_overflow_rows(const uint8_t* codes, int64_t N, int64_t K, int r, int32_t* row_ptr,
                           void* stream);
MQ_API mq_status mq_overflow_cols(const uint8_t* codes, int64_t N, int64_t K, int r,
                           const int32_t* row_ptr, uint16_t* col_idx, void* stream);
MQ_API mq_status mq_overflow_apply(const int32_t* row_ptr, const uint16_t* col_idx, int r,
                            const float* alpha, int64_t group, int64_t N, int64_t K,
                            const uint16_t* x, int64_t M, float* y, void* stream);

/* One matrix of a grouped sparse addition (see mq_overflow_apply_grouped). */
typedef struct mq_overflow_problem {
  const int32_t* row_ptr;  /* int32 [N + 1]                     */
  const uint16_t* col_idx; /* uint16 [row_ptr[N]]              */
  const float* alpha;      /* fp32 [N, K/group]                 */
  const uint16_t* x;       /* bf16 bits [M, K]                  */
  float* y;                /* fp32 [M, N] (updated)             */
  int64_t N, K, group;
} mq_overflow_problem;

/*
 * mq_overflow_apply_grouped: mq_overflow_apply for several matrices at the
 * same r and M in one launch (for example the three matrices of a
 * feed-forward block); same definitions, checks and result per matrix.
 * Outputs must not overlap.  1 <= count <= 16.
 */
MQ_API mq_status mq_overflow_apply_grouped(const mq_overflow_problem* problems, int count, int r,
                                    int64_t M, void* stream);

/*
 * Bit-plane storage: one stored copy of the codes, as eight planes of one bit
 * each, serving every precision r = 1..8 without repacking (the one stored
 * int8 model of the explainer's §2 and "The Bit-Slicing Operator", read by
 * bit).  The index of Eq. 6 is the integer part h of q / 2^(8-r) (planes
 * 8-r .. 7) plus the first discarded bit c (plane 7-r), clamped to 2^r - 1;
 * a server at r reads r + 1 planes, (r + 1)/8 of the bytes (all 8 at r = 8).
 *
 * Layout (uint8 [8][N][K/8], plane p = bit p of q): each plane row is cut
 * into 512-code superblocks of 16 little-endian 32-bit words; word 4s + G
 * holds at bit 16h + i the bit of code 128G + 32s + 2i + h of the superblock
 * (s, G in 0..3, i in 0..15, h in 0..1).
 *
 * mq_bitplanes_bytes: N * K (0 on invalid shapes).
 * mq_pack_bitplanes: codes uint8 [N, K] -> planes (output), both 16-byte
 *   aligned.  Bit-exact.
 * mq_gemv_bitplanes: the product of mq_gemv with the index read from the
 *   planes.  extra = 1 leaves out the clamp (the errata Eq. 8,
 *   Extra-Precision MatQuant: the index may reach 2^r, value 256) and so
 *   needs no overflow lists; at r = 8 it changes nothing.
 *   alpha, zero fp32 [N, K/group]; x bf16 bits [M, K] and y fp32 [M, N],
 *   16-byte aligned.
 * Sizes: N >= 1, K % 512 == 0, 512 <= K <= 65536, N * K <= 2^31;
 * 1 <= M <= 8; 1 <= r <= 8; group = K or 128; extra in {0, 1}.
 */
MQ_API size_t mq_bitplanes_bytes(int64_t N, int64_t K);
MQ_API mq_status mq_pack_bitplanes(const uint8_t* codes, int64_t N, int64_t K, uint8_t* planes,
                            void* stream);
MQ_API mq_status mq_gemv_bitplanes(const uint8_t* planes, int r, int extra, const float* alpha,
                            const float* zero, int64_t group, int64_t N, int64_t K,
                            const uint16_t* x, int64_t M, float* y, void* stream);

/*
 * Mix'n'Match stack ("Matryoshka Quantization" explainer, §3.4 "Mix'n'Match
 * and Interpolative Slicing"): a stack of layers over one stored int8 model,
 * each layer sliced to its own r.
 *
 * Layer dataflow (the pages give none; this is the library's definition):
 *   a = bf16(h / sqrt(mean(h^2)))            (per row, fp32 arithmetic)
 *   q = W_q a, k = W_k a, v = W_v a, u = W_up a, g = W_gate a
 *   o = W_o bf16(q),  d = W_down bf16(u * g)  (u * g in fp32)
 *   h = h + o + d                             (fp32 residual stream)
 * k and v are computed and written to the workspace but not consumed.
 * Shapes: q, o: [H, H]; k, v: [Hkv, H]; up, gate: [F, H]; down: [H, F];
 * the same H, Hkv, F in every layer, H <= 16384 (the norm holds a row in
 * registers; larger H returns MQ_ERR_SHAPE).  Each mq_linear holds the plane
 * packed at its layer's r.
 */
typedef struct mq_linear {
  const uint8_t* packed; /* uint8 [N, K*r/8] at the layer's r */
  const float* alpha;    /* fp32 [N, K/group]                 */
  const float* zero;     /* fp32 [N, K/group]                 */
  int64_t N, K, group;
} mq_linear;

typedef struct mq_layer {
  int r; /* 2, 3, 4, 6 or 8 */
  mq_linear q, k, v, o, up, gate, down;
} mq_layer;

/* Workspace bytes for mq_mixnmatch_forward (0 on invalid shapes). */
MQ_API size_t mq_mixnmatch_workspace_bytes(const mq_layer* layers, int n_layers, int64_t M);

/*
 * Byte offsets inside the workspace of the intermediates of the LAST layer
 * run, valid after the call's work completes: a (bf16 [M, H]), q, k, v
 * (fp32 [M, H] / [M, Hkv]), u, g (fp32 [M, F]), o, d (fp32 [M, H]),
 * bf16(q) (bf16 [M, H]) and bf16(u * g) (bf16 [M, F]; written only when up
 * and gate have the same group, which lets one launch compute both and their
 * product).  offsets must have room for 10 entries, in that order.
 */
MQ_API mq_status mq_mixnmatch_workspace_offsets(const mq_layer* layers, int n_layers, int64_t M,
                                         size_t* offsets);

/*
 * mq_mixnmatch_forward: run n_layers layers on the bf16 input x [M, H]:
 * h = x (exact in fp32), then every layer in order; the final residual
 * stream is written to h_out (fp32 [M, H]).  x and h_out 16-byte aligned and
 * not overlapping.  1 <= M <= 8, 1 <= n_layers.  `layers` is a HOST array
 * read during the call only.
 */
MQ_API mq_status mq_mixnmatch_forward(const mq_layer* layers, int n_layers, const uint16_t* x,
                               int64_t M, float* h_out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * mq_mixnmatch_forward_inplace: the same layers run on an fp32 residual
 * stream h [M, H] that the caller already holds (updated in place), to
 * continue a stack over several calls (a block of layers per call, e.g. one
 * pipeline stage, or one layer at a time): h keeps full fp32 precision
 * between calls, which a bf16 input could not.  Same constraints otherwise.
 */
MQ_API mq_status mq_mixnmatch_forward_inplace(const mq_layer* layers, int n_layers, float* h,
                                       int64_t M, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * Decode MLP block on sliced planes (the FFN, the main decode cost: the
 * explainer's §5; a step either side of the product):
 *   u = W_up x,  g = W_gate x              (one launch: the rows of up and
 *                                           gate share workgroups and x)
 *   a = bf16(u * act(g))                    (fp32 product, nearest even)
 *   y = W_down a                            (second launch)
 * act: 0 identity, 1 SiLU (g * sigmoid(g)), 2 GELU, tanh form.  The pages
 * give no MLP block; this is the library's definition.
 *   up, gate: mq_linear [F, H] (same group); down: mq_linear [H, F]; all
 *   packed at r (r in {2, 3, 4, 6, 8}).
 *   x bf16 bits [M, H] and y fp32 [M, H] (output), 16-byte aligned;
 *   1 <= M <= 8.
 *   workspace: mq_mlp_workspace_bytes(M, F) bytes, 256-byte aligned; after
 *   the call's work it holds u and g (fp32 [M, F]) at byte offsets 0 and A
 *   and a (bf16 [M, F]) at 2A, with A = M*F*4 rounded up to 256.
 * Returns MQ_ERR_GROUP if up and gate differ in group.
 */
MQ_API size_t mq_mlp_workspace_bytes(int64_t M, int64_t F);
MQ_API mq_status mq_mlp_decode(const mq_linear* up, const mq_linear* gate, const mq_linear* down, int r,
                        int act, const uint16_t* x, int64_t M, float* y, void* workspace,
                        size_t workspace_bytes, void* stream);


#ifdef __cplusplus
}
#endif
#endif /* MQ_H */
