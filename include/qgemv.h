/*
 * qgemv.h -- C ABI of libqgemv.so, block-dequant GEMV for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (the decode-time matrix-vector products of the
 * from-scratch LLM engines on the pages):
 *   y[n] = sum_k W[n][k] * x[k],   W[n][k] = d(n, k/32) * v(n, k)
 * where W is read in a GGUF-style block-quantised form and dequantised inside
 * the product ("EdgeRunner beats llama.cpp", What worked, item 2: fused Q8_0
 * dequant + GEMV, no float copy of the weights).
 *   Q8_0: 32 int8 quants + one fp16 scale per block, v = q            (34 B / 32 weights)
 *   Q4_0: 32 4-bit quants + one fp16 scale per block, v = nibble - 8  (18 B / 32 weights)
 * (RunIT_Mac README, optimisation table: 1.06 and 0.56 bytes per weight.)
 * x and y are fp32 and the accumulation is fp32 (RunIT_Mac README, kernel table
 * "f32in_f32out" names and the f32 data-flow figure).
 *
 * Conventions for every call below
 *  - Pointers named *_host are host memory. Every other pointer is DEVICE
 *    memory (hipMalloc / torch CUDA tensors), never a host mapping: the pages
 *    measured running the weights off a memory-mapped file as their worst bug
 *    (robotnurse.io "We wrote our own inference engine", What actually moved it, 1).
 *  - stream is a hipStream_t passed as void*; NULL means the null stream.
 *    Calls only enqueue work and return; results are valid once the caller has
 *    synchronised that stream. Device faults surface at that synchronisation.
 *  - The caller owns and frees every buffer. The GEMV calls allocate nothing
 *    and keep no per-call state; they may be captured into a HIP graph.
 *  - Arguments are checked on the host before any HIP call. A bad argument
 *    returns QG_EINVAL / QG_EALIGN / QG_EUNSUPPORTED and enqueues nothing; a
 *    failed launch returns QG_EHIP. qg_last_error() gives a thread-local
 *    message for the last failure on the calling thread. Order of the checks:
 *    sizes and types, null pointers, alignment, then overlaps.
 *  - Alignment of the quantised GEMV calls (qgemv_q8_0, qgemv_q4_0, qgemv_q4_k,
 *    qgemv_q6_k, qgemv_epilogue, qgemv_fused_gateup_silu, qgemv_verify,
 *    qgemv_rmsnorm, qgemv_rmsnorm_gateup_silu): packed weights, x / X and gamma
 *    16-byte aligned (the kernels read them with 16-byte loads); fp32 outputs,
 *    bias and residual 4-byte aligned; fp16 outputs 2-byte aligned. Anything
 *    less returns QG_EALIGN.
 *  - Same inputs give bitwise the same outputs, run to run (no atomics, no
 *    cross-workgroup reductions, fixed reduction trees).
 *  - Quantised weights are re-tiled once, at load time, by qg_pack* into the
 *    library's packed layout, the way the robotnurse.io post folds projections
 *    once at load rather than per token (What actually moved it, 5). The packed
 *    layout is internal: only qg_packed_size() and the pack/unpack calls know it.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_OK = 0,
    QG_EINVAL = 1,       /* null pointer, bad size, overlapping buffers        */
    QG_EALIGN = 2,       /* a pointer is not aligned as the call requires       */
    QG_EUNSUPPORTED = 3, /* unknown qtype, or M outside 2..6 for verify         */
    QG_EHIP = 4          /* the HIP runtime reported an error at launch         */
} qg_status;

typedef enum { QG_Q8_0 = 1, QG_Q4_0 = 2, QG_Q4_K = 3, QG_Q6_K = 4 } qg_qtype;

/* ---- load-time packing --------------------------------------------------- */

/* Bytes of the packed form of an N x K matrix of `qtype` (K % 32 == 0, K % 256
 * == 0 for QG_Q4_K and QG_Q6_K, N, K > 0).
 * Returns 0 for invalid arguments. The packed form holds the same quant and
 * scale bytes as the canonical one plus zero padding of the last row tile (up
 * to 7 rows) and 256-byte alignment of its two planes (three for Q4_K and
 * Q6_K, whose super-block scales get a plane of their own). */
size_t qg_packed_size(int qtype, int64_t N, int64_t K);

/* Re-tile a canonical matrix already in device memory into the packed layout.
 * canonical: N*K/32 GGUF-style blocks, row-major (row n = K/32 consecutive
 *   blocks; block = little-endian fp16 scale then the quants; Q4_0 byte j holds
 *   element j in its low nibble and element j+16 in its high nibble); for Q4_K
 *   and Q6_K N*K/256 super-blocks of 144 / 210 bytes, laid out as qgemv_q4_k /
 *   qgemv_q6_k state.
 * packed: qg_packed_size(qtype, N, K) bytes, 16-byte aligned, not overlapping
 *   canonical. Padding rows are written as zeros. Stream-ordered kernel. */
qg_status qg_pack(int qtype, const void *canonical, void *packed, int64_t N, int64_t K, void *stream);

/* Load-time concatenation (e.g. Q, K and V projections into one fused QKV
 * weight, RunIT_Mac README "Fused QKV+bias"): pack the nrows canonical rows into
 * rows [row0, row0 + nrows) of a packed N_total x K matrix. The call whose rows
 * end at N_total also zero-fills the padding rows. Calls for disjoint row
 * ranges may run in any order. */
qg_status qg_pack_rows(int qtype, const void *canonical, void *packed, int64_t N_total,
                       int64_t row0, int64_t nrows, int64_t K, void *stream);

/* Load-time fusion of a gate and an up projection (each N_ff x K, canonical,
 * device memory) into one packed weight for qgemv_fused_gateup_silu.
 * packed: qg_packed_size(qtype, 2 * N_ff, K) bytes, 16-byte aligned.
 * Gate row n and up row n are placed in the same wavefront's registers. */
qg_status qg_pack_gateup(int qtype, const void *gate, const void *up, void *packed,
                         int64_t N_ff, int64_t K, void *stream);

/* Host-memory versions of the packer and its inverse (same bytes as the device
 * packer). unpack(pack(B)) == B byte for byte. gate/up fusion on the host:
 * qg_pack_gateup_host. */
qg_status qg_pack_host(int qtype, const void *canonical_host, void *packed_host, int64_t N, int64_t K);
qg_status qg_unpack_host(int qtype, const void *packed_host, void *canonical_host, int64_t N, int64_t K);
qg_status qg_pack_gateup_host(int qtype, const void *gate_host, const void *up_host, void *packed_host,
                              int64_t N_ff, int64_t K);

/* ---- the GEMVs ----------------------------------------------------------- */

/* y[N] = W x for a packed Q8_0 weight (N x K, K % 32 == 0); x: fp32 [K];
 * y: fp32 [N]. w_packed and x 16-byte aligned, y 4-byte aligned; y must not
 * overlap x or w_packed. A fused QKV projection is this call on the packed
 * concatenation (qg_pack_rows); the caller slices y. */
qg_status qgemv_q8_0(const void *w_packed, const float *x, float *y, int64_t N, int64_t K, void *stream);

/* Same for a packed Q4_0 weight (weight value nibble - 8), with the same
 * alignment (w_packed and x 16 bytes, y 4 bytes). */
qg_status qgemv_q4_0(const void *w_packed, const float *x, float *y, int64_t N, int64_t K, void *stream);

/* The same for a packed Q4_K weight (K % 256 == 0). Q4_K is the k-quant block
 * of the RunIT_Mac README's "Fused Q4_K dequant + GEMV" kernel and Q4_K_M
 * models (quantisation table); its layout is not on the pages and is read as
 * the published GGUF block: per 256 weights an fp16 d and dmin, eight 6-bit
 * sub-block scales sc and mins mn in 12 bytes, 128 bytes of 4-bit quants q;
 * weight = d * sc * q - dmin * mn. Per 32-weight sub-block the product is
 * summed in fp32 as d*sc * sum((q - c) x) + (d*sc*c - dmin*mn) * sum(x), with
 * c = dmin*mn / (d*sc) rounded and clamped to 0..15, which the packer derives at
 * load time: both terms are bounded by 3 |w| per weight, so each output is
 * within 1e-5 * sum |w x| + 1e-7 of the exact product like the other types,
 * also where d*sc*q and dmin*mn cancel. Same alignment as qgemv_q4_0.
 * Q4_K packs with qg_pack / qg_pack_rows / qg_pack_gateup / qg_pack_host (148
 * bytes per 256 weights). The other GEMV calls (qgemv_epilogue,
 * qgemv_fused_gateup_silu, qgemv_verify, qgemv_rmsnorm,
 * qgemv_rmsnorm_gateup_silu) take it as qtype QG_Q4_K, with the same sums; the
 * prefill GEMM returns QG_EUNSUPPORTED for it. */
qg_status qgemv_q4_k(const void *w_packed, const float *x, float *y, int64_t N, int64_t K, void *stream);

/* The same for a packed Q6_K weight (K % 256 == 0). Q6_K is the k-quant block
 * the RunIT_Mac README's quantisation table lists as supported and the
 * EdgeRunner page ("Run it yourself") loads; its layout is not on the pages and
 * is read as the published GGUF block: per 256 weights 128 bytes ql of low
 * 4-bit parts, 64 bytes qh of high 2-bit parts, 16 int8 scales sc (one per 16
 * weights), then fp16 d. Weight i (half h = i/128, g = (i%128)/32, l = i%32):
 * q = (low (g < 2) or high nibble of ql[64h + 32(g%2) + l]) | (bits 2g..2g+1 of
 * qh[32h + l]) << 4, weight = d * sc[i/16] * (q - 32). The quants are dequantised
 * exactly (fp16 q - 32) and each 16-weight sum is scaled by its sc, then d.
 * Packs with qg_pack / qg_pack_rows / qg_pack_gateup / qg_pack_host (210 bytes
 * per 256 weights, as canonical); like Q4_K it is taken by every other GEMV
 * call (qtype QG_Q6_K) but not by the prefill GEMM. */
qg_status qgemv_q6_k(const void *w_packed, const float *x, float *y, int64_t N, int64_t K, void *stream);

/* Output element type of qgemv_epilogue. */
typedef enum { QG_OUT_F32 = 0, QG_OUT_F16 = 1 } qg_out_type;

/* Epilogue variants of the M=1 quantised GEMV, in the same dispatch:
 *   y[n] = ((W x)[n] + bias[n]) + residual[n]
 * The RunIT_Mac README adds the QKV bias inside the fused QKV kernel ("Fused
 * QKV+bias", optimisation and kernel tables) and keeps an f32 residual stream
 * that the projections add into (data-flow figure); the robotnurse.io post
 * lists fp16-output GEMVs among its wins (What actually moved it, 5).
 *  - qtype QG_Q8_0 / QG_Q4_0; w_packed from qg_pack / qg_pack_rows (16-byte
 *    aligned); x fp32 [K] (16-byte aligned).
 *  - (W x)[n] has exactly the bits that qgemv_q8_0 / qgemv_q4_0 return. Each
 *    addition is one fp32 add, bias first; a NULL bias or residual is skipped,
 *    so with both NULL and QG_OUT_F32 this call equals the plain one.
 *  - bias, residual: fp32 [N], 4-byte aligned, or NULL.
 *  - out_type QG_OUT_F32: y is fp32 [N] (4-byte aligned). QG_OUT_F16: y is
 *    fp16 [N] (2-byte aligned), the fp32 result rounded to nearest even
 *    (subnormals kept, overflow to infinity).
 *  - residual may be the same buffer as y (in-place y += W x) with QG_OUT_F32;
 *    any other overlap of y with x, the weights, bias or residual returns
 *    QG_EINVAL. An unknown out_type returns QG_EUNSUPPORTED. */
qg_status qgemv_epilogue(int qtype, const void *w_packed, const float *x, const float *bias,
                         const float *residual, void *y, int out_type, int64_t N, int64_t K, void *stream);

/* Unquantised fp16 weights, y = W x with W fp16 row-major [N][K] (any K >= 1,
 * 2-byte aligned), x fp32 [K] (4-byte aligned), y fp32 [N] (4-byte aligned,
 * not overlapping x or W). Each row's K is split, and the partial sums are
 * combined in a fixed order: deterministic, no workspace, no atomics
 * (robotnurse.io post, What actually moved it, 4: a split-K fp16 GEMV for the
 * unquantised matrices). Forms, chosen by shape; the first two need K % 8 == 0
 * and W and x 16-byte aligned, else the last form runs:
 *  - fewer than 1024 rows and K <= 32768: one workgroup per row, K split into
 *    consecutive ranges over up to 16 wavefronts, partials added in wavefront
 *    order;
 *  - otherwise, K = 512 L with L <= 16: one wavefront per row, K split over its
 *    64 lanes, with the whole row's loads in flight at once;
 *  - otherwise: one workgroup per row, K split over the lanes of one wavefront
 *    (four below 1024 rows) in 8-element chunks, partials added in wavefront
 *    order. */
qg_status gemv_f16_splitk(const void *w_f16, const float *x, float *y, int64_t N, int64_t K, void *stream);

/* Fused gate+up with the SiLU epilogue (RunIT_Mac README "Fused gate+up+silu",
 * one dispatch instead of three): y[n] = silu(g[n]) * u[n] for n < N_ff, where
 * g = W_gate x, u = W_up x and silu(g) = g / (1 + exp(-g)).
 * w_gateup_packed comes from qg_pack_gateup (16-byte aligned); x fp32 [K]
 * (16-byte aligned); y fp32 [N_ff] (4-byte aligned, not overlapping x or the
 * weights). */
qg_status qgemv_fused_gateup_silu(int qtype, const void *w_gateup_packed, const float *x, float *y,
                                  int64_t N_ff, int64_t K, void *stream);

/* RMSNorm of one activation vector (RunIT_Mac README, kernel table and
 * data-flow figure: f32 input, f32 gamma, f32 output):
 *   out[k] = (x[k] * r) * gamma[k],   r = 1 / sqrt(sum_j x[j]^2 / K + eps)
 * in fp32: the sum of squares is a fixed-order reduction (deterministic), the
 * square root and the division are correctly rounded. One workgroup. x, gamma,
 * out fp32 [K] (K >= 1), 4-byte aligned; out must not overlap x or gamma; eps
 * finite and >= 0 (the pages give no value; Qwen-style models use 1e-6). This
 * is the unfused form of the prologue below. */
qg_status qg_rmsnorm(const float *x, const float *gamma, float eps, float *out, int64_t K, void *stream);

/* GEMV with the RMSNorm of its activation fused into the prologue ("EdgeRunner
 * beats llama.cpp", The progression: RMSNorm+GEMV kernel fusion; the
 * robotnurse.io post, Things that lost, measured the same fusion as a loss from
 * L2 re-reads per threadgroup): y = W * rmsnorm(x), one dispatch. Every
 * workgroup stages x in LDS, reduces sum(x^2) itself and normalises its copy,
 * then runs the GEMV of qgemv_q8_0 / qgemv_q4_0 on it. Arguments as for those
 * calls (w_packed and x 16-byte aligned, y 4-byte aligned) plus gamma fp32 [K]
 * (16-byte aligned, not overlapping y) and eps as in
 * qg_rmsnorm. K <= 39936 (the normalised copy lives in LDS, next to the
 * kernel's own static arrays), else QG_EUNSUPPORTED. The result is within the linear tolerance of the exact
 * product on the exact normalised vector; it is not bitwise equal to
 * qg_rmsnorm followed by the plain GEMV (another reduction order). */
qg_status qgemv_rmsnorm(int qtype, const void *w_packed, const float *x, const float *gamma, float eps, float *y,
                        int64_t N, int64_t K, void *stream);

/* The fused gate|up SiLU GEMV with the same RMSNorm prologue:
 * y[n] = silu(g[n]) * u[n], g = W_gate * rmsnorm(x), u = W_up * rmsnorm(x). */
qg_status qgemv_rmsnorm_gateup_silu(int qtype, const void *w_gateup_packed, const float *x, const float *gamma,
                                    float eps, float *y, int64_t N_ff, int64_t K, void *stream);

/* Multi-row "verify" GEMV: Y[m][n] = sum_k W[n][k] X[m][k] for 2 <= M <= 6,
 * X fp32 row-major [M][K] (16-byte aligned; K % 32 == 0 keeps every row
 * 16-byte aligned), Y fp32 row-major [M][N] (4-byte aligned, not overlapping
 * X or the weights), w_packed 16-byte aligned. The packed weights are
 * streamed once for all M rows (on a matrix with so few row tiles that one
 * pass would leave most of the chip idle, the rows are split into groups
 * that each read the weights, the later reads mostly from the caches), and
 * row m of Y is bit-for-bit (memcmp) equal
 * to what qgemv_q8_0 / qgemv_q4_0 return for x = X[m] (robotnurse.io post,
 * Update and "Correctness first": a 3-6-row verify pass in one weight stream,
 * checked against the decode kernel with memcmp). */
qg_status qgemv_verify(int qtype, const void *w_packed, const float *X, float *Y,
                       int64_t N, int64_t K, int M, void *stream);

/* ---- small-M GEMM (prefill chunks) ---------------------------------------- */

/* Bytes of the workspace qgemm_prefill needs for this weight shape and M
 * activation rows (0 for invalid arguments): per-row factors, the split
 * activations (M rounded up to 16, times K times 4 bytes) and, when the launch
 * plan splits K across workgroups, ksplit * M * N partial sums. The plan
 * depends on the current device's CU count: query on the device that runs the
 * call. */
size_t qg_prefill_workspace_size(int qtype, int64_t N, int64_t K, int64_t M);

/* Y = X W^T for a chunk of M activation rows against a packed Q8_0 / Q4_0
 * weight, on the matrix cores: Y[m][n] = sum_k W[n][k] X[m][k], the dense side
 * of the same weights (RunIT_Mac README, roadmap and source tree: "Prefill
 * batching (GEMM kernel)"; the robotnurse.io post prefills in 128-token
 * chunks). X fp32 row-major [M][K], Y fp32 row-major [M][N], 1 <= M <= 2^20,
 * both 4-byte aligned; w_packed from qg_pack (16-byte aligned).
 * workspace: caller-owned device memory of
 * qg_prefill_workspace_size(qtype, N, K, M) bytes, 256-byte aligned, overlapping nothing else; it holds the activations
 * split into two fp16 parts (one power-of-two scale per row, 22 significant
 * bits) and the partial sums of a K split, and is overwritten by every call.
 * The weights are streamed once per 64 (Q8_0) or 32 (Q4_0) activation rows; matrices with few row
 * tiles split K across workgroups and add the ranges in a fixed order. Each
 * output is within 1e-5 * sum_k |W[n][k] X[m][k]| + 1e-7 of the exact product
 * for finite inputs; it is deterministic but not bitwise equal to qgemv_q8_0
 * / qgemv_q4_0 / qgemv_verify (another order of additions). Kernels enqueued:
 * the split, the GEMM passes and, with a K split, the sum of the ranges;
 * qg_time_next_launch times the first GEMM pass. */
qg_status qgemm_prefill(int qtype, const void *w_packed, const float *X, float *Y, int64_t N, int64_t K, int64_t M,
                        void *workspace, size_t workspace_bytes, void *stream);

/* The same GEMM for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument. Its scratch (the split activations, row factors and
 * K-range partials that qgemm_prefill keeps in the caller's workspace) is one
 * file-scope device array of QG_PREFILL_NOALLOC_MAX_BYTES (64 MiB) per GPU,
 * held by the library until the process ends; the first call on each device
 * takes the array's device address (hipGetSymbolAddress). The call allocates
 * and frees nothing. A shape whose workspace (qg_prefill_workspace_size) is
 * larger returns QG_EUNSUPPORTED before any HIP call. Every call on a GPU
 * shares that GPU's array, which keeps the last call's contents (each call
 * writes every scratch byte it reads first): calls that overlap in time on
 * one GPU race, so issue them on one stream or otherwise serialise them.
 * Arguments and results as for qgemm_prefill: Y is bit for bit what
 * qgemm_prefill returns with a workspace. */
#define QG_PREFILL_NOALLOC_MAX_BYTES ((size_t)64 << 20)
qg_status qgemm_prefill_noalloc(int qtype, const void *w_packed, const float *X, float *Y, int64_t N, int64_t K,
                                int64_t M, void *stream);

/* ---- diagnostics --------------------------------------------------------- */

const char *qg_status_str(int status);
const char *qg_last_error(void);

/* How a quantised call of this shape is launched (for reports and tests).
 * Inputs: qtype, N, K as for the GEMV calls; M activation rows (1..6);
 * rmsnorm 1 for the RMSNorm-prologue calls (M = 1 only), else 0.
 * Outputs (each may be NULL):
 *   split_k_ways  the number of K ranges a row tile's sum is split into (the
 *                 partial sums of a row are added in range order);
 *   workgroups    workgroups launched (a verify call on a matrix with few row
 *                 tiles splits its M rows into groups, each group its own set
 *                 of workgroups: this counts them all);
 *   x_in_lds      1 when the activations are staged in LDS, 0 when read from L2;
 *   persistent    1 for the persistent form (one workgroup per CU, used for
 *                 matrices with few row tiles), 0 for one wavefront per tile;
 *   lds_bytes     LDS per workgroup, static arrays plus the dynamic part (at
 *                 most the 160 KiB of a gfx950 CU).
 * Host function: it only reads the current device's CU count (256 when no
 * device answers). Returns QG_OK, QG_EINVAL, or QG_EUNSUPPORTED where the
 * call itself would (M outside 1..6; rmsnorm with M != 1, K > 39936, or
 * activations that do not fit in LDS). */
qg_status qg_plan_info(int qtype, int64_t N, int64_t K, int M, int rmsnorm, int *split_k_ways,
                       int64_t *workgroups, int *x_in_lds, int *persistent, int64_t *lds_bytes);

/* How gemv_f16_splitk launches for this shape (for reports and tests). w_f16
 * and x are only inspected for their 16-byte alignment, never read. Outputs
 * (each may be NULL): form 2 = one workgroup per row with K split over its
 * wavefronts, 1 = one wavefront per row, 0 = K split over the lanes of one or
 * four wavefronts per row (the three forms of gemv_f16_splitk, in its order);
 * waves = wavefronts per row (form 2, 0) or rows per workgroup (form 1);
 * workgroups launched. Host function. Returns QG_OK or QG_EINVAL. */
qg_status qg_f16_plan_info(int64_t N, int64_t K, const void *w_f16, const float *x, int *form, int *waves,
                           int64_t *workgroups);

/* Measurement kernels (diagnostics; no GEMV uses them).
 * qg_probe_stream: a plain streaming read of `bytes` bytes of device memory
 * (a positive multiple of 1024; buf 16-byte aligned) with 16-byte nontemporal
 * loads, each wavefront reading 8 KiB as 8 one-KiB load instructions issued at
 * once, as the GEMV kernels stream their weights: what the device streams at
 * that size, the ceiling a GEMV's weight stream is held against. `sink`
 * (4 bytes of device memory, not overlapping buf) is written only if the XOR
 * of the words read equals a fixed value, so in practice nothing is written.
 * qg_probe_empty: an empty kernel (one wavefront): the floor of any dispatch.
 * Both are stream-ordered, take qg_time_next_launch timing events, and return
 * QG_OK, QG_EINVAL, QG_EALIGN or QG_EHIP. */
qg_status qg_probe_stream(const void *buf, size_t bytes, uint32_t *sink, void *stream);
qg_status qg_probe_empty(void *stream);

/* Re-read the launch-shape overrides (QG_SPLIT_K, QG_PERSIST, QG_X_GLOBAL,
 * QG_TILES_PER_GROUP, QG_WAVES_PER_WG, QG_PREFETCH, QG_F16_ROWS, QG_F16_WAVES,
 * QG_STRIDE_GROUPS, QG_GEMM_MT, QG_GEMM_WAVES, QG_GEMM_ROWGROUPS, QG_GEMM_KSPLIT,
 * QG_F16_FORM, QG_F16_CPL)
 * from the environment. They exist for launch-shape sweeps and tests and are
 * read once, at the first call that plans a launch; the GEMV calls themselves
 * read no environment. An override that changes a matrix's K split (QG_SPLIT_K,
 * QG_PERSIST) changes its rows' rounding, so it must hold for the decode and
 * the verify call alike. Not safe to call while another thread plans a launch
 * with different overrides in effect. Returns QG_OK. */
qg_status qg_reload_tuning(void);

/* Time the next kernel that the calling thread launches through qgemv_q8_0,
 * qgemv_q4_0, qgemv_epilogue, qgemv_rmsnorm, qgemv_rmsnorm_gateup_silu,
 * qg_rmsnorm, gemv_f16_splitk, qgemv_fused_gateup_silu, qgemv_verify or
 * qgemm_prefill (its first GEMM pass).
 * start_event and stop_event are hipEvent_t handles, created by the caller
 * with timing enabled and owned by the caller. That call's kernel records its
 * own start and end time into them (the dispatch's timestamps, which a
 * kernel trace also reports), so hipEventElapsedTime(start, stop) gives the
 * kernel's duration without the latency of event records queued around it.
 * The setting is used by one call and then cleared; a call that fails, or
 * (NULL, NULL), clears it too. Pack calls neither use nor clear it.
 * Returns QG_OK, or QG_EINVAL when exactly one event is NULL. */
qg_status qg_time_next_launch(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
