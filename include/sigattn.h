/*
 * sigattn.h - C ABI of the MI355X (gfx950) padded sigmoid-attention library.
 *
 * Operation (per batch entry b with n = seqlens[b] valid tokens, per head h):
 *
 *   x_ij  = s * (q_i . k_j) + beta_b [+ log(g_j + eps)]        i, j < n
 *   P_ij  = 1 / (1 + e^{-x_ij})   if key j is kept and (not causal or j <= i), else 0
 *   O_i   = sum_j P_ij * V'_j,    V'_j = g_j * v_j when gated, else v_j
 *
 * with s = 1/sqrt(d) and beta_b = -ln(n). Sources: "Better Models, Faster Training:
 * Sigmoid Attention for single-cell Foundation Models" (arXiv 2604.27124), section 3
 * "Sigmoid Attention" equation (element-wise sigmoid of the scaled scores plus a bias,
 * times V) and section 4 (block-sparse skipping of padded blocks, backward split into a
 * dQ pass and a dK/dV pass with recomputation); its gist.science summary, section 2A,
 * for sigma(x) = 1/(1+e^-x) and b = -log(n); and "Sigmoid Attention as a Better
 * Substrate for Learned KV Cache Eviction" (arXiv 2608.23296), gate paragraphs, for
 * the per-key gate (log g on the logits, g on the values, eps = 1e-8), the hard-drop
 * rule g_j < tau and the leading positions that are never removed.
 *
 * Backward, from the diagonal Jacobian of the element-wise sigmoid (first paper,
 * appendix A.1.2), given dO:
 *   dV_j = g_j sum_i P_ij dO_i          dS_ij = (dO_i . V'_j) * P_ij (1 - P_ij)
 *   dQ_i = s sum_j dS_ij k_j            dK_j  = s sum_i dS_ij q_i
 *
 * Conventions shared by every entry point:
 *  - Tensors q, k, v, o, dO, dq, dk, dv are [B][H][Lmax][d] views described by the
 *    element strides stride_b, stride_h, stride_l (the last dimension is contiguous);
 *    all of them use the same strides, counted in elements of their own type. Input
 *    type (q, k, v, dO): bf16 (SIGATTN_BF16) or float (SIGATTN_F32, a slow debug
 *    path). Output type (o, dq, dk, dv): out_dtype, bf16 or float; float inputs
 *    require float outputs. Accumulation is always float.
 *  - Precision of the bf16 path. The attention weights P and the score gradients dS
 *    are formed in float and enter the second product of each pass as bf16 operands
 *    of the matrix cores. With fast_math = 0 (the default) each is carried as an
 *    unevaluated sum hi + lo of two bf16 values (about 16 significant bits; two
 *    matrix-core products instead of one), so that the result is limited by the
 *    bf16 inputs and the output type only. With fast_math = 1 a single bf16 value is
 *    used (relative rounding 2^-9 per weight) and the products cost half as much.
 *    fast_math = 2 is the default's backward with an f16 forward: P is rounded once to
 *    f16 (relative 2^-11; kept as 2^14 P, so normal down to P = 2^-28) and multiplied
 *    with V converted to f16 (exact for |v| < 2^16; an item whose V holds a larger value
 *    is computed again on hi + lo operands). Its error in an output row is about 2^-11
 *    of that row's size, which meets max|err|/rms <= 2e-2 over a batch whose rows are of
 *    similar size, but not over one that mixes sequences of very different lengths (a
 *    row of a 2-token sequence next to those of an 8192-token one) or holds a few rows
 *    much larger than the rest.
 *  - seqlens and bias are HOST arrays of length B, read during the call only.
 *    gate is a DEVICE array of floats, gate[b * gate_stride_b + j], j < Lmax.
 *  - The caller owns every buffer. The library never allocates, frees or
 *    synchronises; only sigattn_decode needs a workspace, which the caller passes
 *    (sigattn_decode_noalloc uses a static device array of the library instead).
 *    Work is enqueued on `stream` (a hipStream_t; NULL is the default stream) and the
 *    results are valid once that stream has completed it. Identical inputs give
 *    bitwise-identical outputs (no atomics).
 *  - Outputs are fully written: rows i >= n of O and dQ, rows j >= n of dK and dV,
 *    and the dK/dV rows of dropped keys are exactly 0. Values in padded input slots
 *    are never read. Inputs are not modified; outputs must not alias inputs.
 *  - Arguments are checked on the host before anything is enqueued. On any error the
 *    call returns a non-zero status and enqueues nothing. A failed launch returns
 *    SIGATTN_ERR_HIP (from hipGetLastError; no synchronisation).
 *  - Every function is thread-safe, never aborts and never prints.
 */
#ifndef SIGATTN_H
#define SIGATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SIGATTN_VERSION 2
#define SIGATTN_MAX_BATCH 256      /* B above this returns SIGATTN_ERR_UNSUPPORTED */
#define SIGATTN_MAX_LEN 65535      /* Lmax above this returns SIGATTN_ERR_UNSUPPORTED */
#define SIGATTN_MAX_ROW_STRIDE (1 << 22)  /* stride_l above this (elements): UNSUPPORTED */
/* Work items of one pass (128-row query or key tiles, summed over sequences and heads;
 * packed batches: B * H * ceil(max rows / 128)) above this return
 * SIGATTN_ERR_UNSUPPORTED: one launch holds at most 2^32 - 1 work-items of 256 threads,
 * and sigattn_bwd puts two passes into one launch. */
#define SIGATTN_MAX_ITEMS ((1 << 23) - 1)

typedef enum {
  SIGATTN_OK = 0,
  SIGATTN_ERR_INVALID_ARG = 1,   /* NULL pointer, bad size, length out of range, aliasing */
  SIGATTN_ERR_UNSUPPORTED = 2,   /* d not in {64,128}, B or Lmax above the caps, dtypes */
  SIGATTN_ERR_ALIGNMENT = 3,     /* a base pointer or a row stride is not 16-byte aligned */
  SIGATTN_ERR_HIP = 4            /* the HIP runtime reported an error at launch */
} sigattn_status;

typedef enum { SIGATTN_BF16 = 0, SIGATTN_F32 = 1 } sigattn_dtype;

typedef struct sigattn_problem {
  uint32_t struct_size;          /* sizeof(sigattn_problem): ABI check */
  int32_t B, H, Lmax, d;         /* 0 <= B <= 256, H >= 1, 1 <= Lmax <= 65535, d in {64,128} */
  int32_t dtype;                 /* sigattn_dtype of q, k, v, dO */
  int32_t out_dtype;             /* sigattn_dtype of o, dq, dk, dv (F32 when dtype is F32) */
  int32_t fast_math;             /* 0: hi+lo split operands (default); 1: single bf16;
                                     2: f16 P V in the forward, hi+lo in the backward */
  int64_t stride_b, stride_h, stride_l;  /* element strides, >= 0; d <= stride_l <= 2^22 */
  const int32_t* seqlens;        /* HOST [B]: valid length n_b, 0 <= n_b <= Lmax */
  int32_t causal;                /* 0: bidirectional; 1: key j allowed for query i iff j <= i */
  float scale;                   /* s; 0 selects 1/sqrt(d) */
  const float* bias;             /* HOST [B] or NULL: NULL selects beta_b = -ln(n_b) */
  const float* gate;             /* DEVICE floats or NULL (no gate) */
  int64_t gate_stride_b;         /* elements between batch rows of gate; 0 selects Lmax */
  float gate_eps;                /* added inside the log: 1e-8 in the pages; >= 0 */
  float gate_tau;                /* key j dropped iff j >= gate_sink and g_j < gate_tau */
  int32_t gate_sink;             /* leading positions never dropped (4 in the pages) */
} sigattn_problem;

/* Check a problem description on the host; touches no GPU. */
sigattn_status sigattn_validate(const sigattn_problem* p);

/* Forward: o = sigmoid attention of (q, k, v). Rows i >= n_b of o are written as 0.
 * Paper: section 3 equation; fully padded query and key tiles are never computed
 * (section 4, block-sparse computation). */
sigattn_status sigattn_fwd(const sigattn_problem* p, const void* q, const void* k,
                           const void* v, void* o, void* stream);

/* Forward plus the row mass of every query: row_mass[b][h][i] = sum_j P_ij over the
 * allowed keys of query i (the attention weights, with the gate's log term in the
 * logits but without the value factor g_j). Without row normalisation this total is
 * free to vary from query to query ("Sigmoid Attention as a Better Substrate for
 * Learned KV Cache Eviction", row-sum diagnostic); its spread across queries is what
 * that diagnostic reports. o is exactly that of sigattn_fwd.
 *  row_mass  DEVICE float [B][H][Lmax], dense (entry (b,h,i) at (b*H + h)*Lmax + i),
 *            4-byte aligned, fully written: 0 for i >= n_b. Must not alias another
 *            argument. */
sigattn_status sigattn_fwd_rowsum(const sigattn_problem* p, const void* q, const void* k,
                                  const void* v, void* o, float* row_mass, void* stream);

/* Backward, query side: dq = s sum_j dS_ij k_j, recomputing P (no stored attention).
 * Rows i >= n_b of dq are written as 0. Paper: section 4, backward decomposition. */
sigattn_status sigattn_bwd_dq(const sigattn_problem* p, const void* q, const void* k,
                              const void* v, const void* dout, void* dq, void* stream);

/* Backward, key side: dk = s sum_i dS_ij q_i and dv = g_j sum_i P_ij dO_i, recomputing
 * P; each key row is owned by one workgroup, so no atomics are used. Rows j >= n_b and
 * rows of dropped keys are written as 0. Paper: section 4, backward decomposition. */
sigattn_status sigattn_bwd_dkdv(const sigattn_problem* p, const void* q, const void* k,
                                const void* v, const void* dout, void* dk, void* dv,
                                void* stream);

/* The whole backward in one call: dq as sigattn_bwd_dq, dk and dv as sigattn_bwd_dkdv,
 * bitwise the same values (the same two kernels' arithmetic; paper: section 4, backward
 * decomposition, one kernel per side, no atomics). At d = 64 with bf16 inputs both
 * kernels' work items go into one launch, so that each pass's last, shorter items share
 * the GPU with the other pass's work instead of leaving it partly idle; otherwise the two
 * passes are enqueued one after the other. Arguments and errors as for the two calls;
 * dq, dk and dv must be distinct and alias no input. */
sigattn_status sigattn_bwd(const sigattn_problem* p, const void* q, const void* k,
                           const void* v, const void* dout, void* dq, void* dk, void* dv,
                           void* stream);

/* Backward, key side, plus the gradient of the per-key gate (requires p->gate).
 * g_j enters twice, as log(g_j + eps) on the logits and as the factor g_j on v_j; by the
 * chain rule (diagonal Jacobian as above) the derivative of sum(dO * O) over head h is
 *   dg_head[b][h][j] = sum_i dS_ij / (g_j + eps) + v_j . sum_i P_ij dO_i
 * ("Sigmoid Attention as a Better Substrate for Learned KV Cache Eviction", gate
 * paragraphs: the gates are trained with the model). dk and dv are exactly those of
 * sigattn_bwd_dkdv.
 *  dg_head  DEVICE float [B][H][Lmax], dense (entry (b,h,j) at (b*H + h)*Lmax + j),
 *           4-byte aligned, fully written: 0 for j >= n_b and for dropped keys (the
 *           drop is a step in g, derivative 0).
 *  dg       DEVICE float [B][Lmax], dense, or NULL: the gradient of the gate shared by
 *           the heads, dg[b][j] = sum over h of dg_head[b][h][j], summed in head order
 *           (deterministic). 4-byte aligned.
 * Neither may alias another argument. Returns SIGATTN_ERR_INVALID_ARG without a gate. */
sigattn_status sigattn_bwd_dkdv_dg(const sigattn_problem* p, const void* q, const void* k,
                                   const void* v, const void* dout, void* dk, void* dv,
                                   float* dg_head, float* dg, void* stream);

/* ------------------------- packed variable-length batches ---------------------------
 *
 * Sequences packed back to back without padding, their bounds in DEVICE arrays (so that a
 * data loader or a previous kernel can produce them without a host round trip), query
 * and key lengths that may differ, and no cap on B. Sequence b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q, o, dO, dq and key rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k, v, dk, dv; nq_b and nk_b are the
 * differences. Every packed tensor is [rows][H][d] with element (t, h, c) at
 * t * stride_t + h * stride_h + c. The operation per (b, h) is that of the padded entry
 * points with n replaced by nq_b for queries and nk_b for keys; the bias defaults to
 * beta_b = -ln(nk_b). Causal alignment is bottom right: key j is allowed for query i iff
 * j <= i + nk_b - nq_b, so a query shard of rows s .. s+m-1 of a causal sequence, given
 * the keys 0 .. s+m-1 and the sequence's bias, yields exactly those rows of the full
 * result: the per-GPU share of context parallelism (outputs of key shards add up,
 * there is no row maximum to merge). All query rows of every sequence are written (rows
 * with no allowed key get 0), and all key rows of dk and dv; rows outside
 * cu[0] .. cu[B]-1 are not touched. Only bf16 inputs; the row-mass and gate-gradient
 * side outputs are not offered here.
 */
typedef struct sigattn_varlen {
  uint32_t struct_size;          /* sizeof(sigattn_varlen): ABI check */
  int32_t B, H, d;               /* B >= 0, H >= 1, d in {64,128} */
  int32_t max_seqlen_q;          /* HOST bound: every nq_b <= max_seqlen_q (sizes the grid) */
  int32_t max_seqlen_k;          /* HOST bound: every nk_b <= max_seqlen_k */
  int32_t out_dtype;             /* sigattn_dtype of o, dq, dk, dv */
  int32_t fast_math;             /* as in sigattn_problem */
  int64_t stride_t, stride_h;    /* element strides of rows and heads, shared by all tensors */
  const int32_t* cu_seqlens_q;   /* DEVICE int32 [B + 1], non-decreasing */
  const int32_t* cu_seqlens_k;   /* DEVICE int32 [B + 1], non-decreasing */
  int32_t causal;                /* 0 or 1 (bottom-right aligned) */
  float scale;                   /* s; 0 selects 1/sqrt(d) */
  const float* bias;             /* DEVICE float [B] or NULL (beta_b = -ln(nk_b)) */
  const float* gate;             /* DEVICE float per packed key row (gate[cu_k[b] + j]) or NULL */
  float gate_eps;
  float gate_tau;
  int32_t gate_sink;
} sigattn_varlen;

/* The bounds in cu_seqlens_q/k are read by the kernels and are not checked on the host;
 * a sequence longer than max_seqlen_q (queries) or max_seqlen_k (keys) is computed only
 * up to that bound. Returns SIGATTN_ERR_UNSUPPORTED when B * H * ceil(max / 128)
 * exceeds SIGATTN_MAX_ITEMS for a pass. sigattn_bwd_varlen computes dq, dk and dv as the
 * two backward calls do, bitwise the same, from one launch at d = 64 (as sigattn_bwd);
 * dq, dk and dv must be distinct and alias no input. */
sigattn_status sigattn_fwd_varlen(const sigattn_varlen* p, const void* q, const void* k,
                                  const void* v, void* o, void* stream);
sigattn_status sigattn_bwd_dq_varlen(const sigattn_varlen* p, const void* q, const void* k,
                                     const void* v, const void* dout, void* dq, void* stream);
sigattn_status sigattn_bwd_dkdv_varlen(const sigattn_varlen* p, const void* q,
                                       const void* k, const void* v, const void* dout,
                                       void* dk, void* dv, void* stream);
sigattn_status sigattn_bwd_varlen(const sigattn_varlen* p, const void* q, const void* k,
                                  const void* v, const void* dout, void* dq, void* dk, void* dv,
                                  void* stream);

/* ------------------- KV cache with threshold eviction, single-query decode -------------------
 *
 * "Sigmoid Attention as a Better Substrate for Learned KV Cache Eviction", gate paragraphs:
 * at inference the soft gate becomes physical deletion. After prefill, entries with
 * g_j < gate_tau are removed; every entry written during decode is kept or removed by the
 * same rule when it is written; positions below gate_sink are never removed; kept entries
 * keep log(g_j + eps) on their logits and g_j on their values. A cache holds only kept
 * entries, in position order, in slots 0..count_b-1; slots at or past count_b hold
 * unspecified values and are never read. The counters live in device memory and are
 * updated by the kernels, so no gate value ever has to travel to the host.
 *
 * A decode step for a new token: write its entry with sigattn_cache_append (kept or not
 * by the rule), then sigattn_decode lets its query attend to the whole cache; a dropped
 * new entry is therefore not seen even by its own query, exactly as a dropped key is
 * masked for every query of the forward. With the bias of the forward, decoding query i
 * against the cache of tokens 0..i reproduces row i of the causal forward.
 */
typedef struct sigattn_cache {
  uint32_t struct_size;          /* sizeof(sigattn_cache): ABI check */
  int32_t B, H, d, cap;          /* 0 <= B <= 256, H >= 1, d in {64,128}, 1 <= cap <= 2^24 */
  int64_t stride_b, stride_h, stride_l;  /* element strides of k and v; d <= stride_l <= 2^22 */
  void* k;                       /* DEVICE bf16 [B][H][cap][d] cached keys */
  void* v;                       /* DEVICE bf16 [B][H][cap][d] cached values */
  float* gate;                   /* DEVICE float [B][cap] gates of the cached entries, or NULL
                                    for a cache without gates (nothing is ever removed) */
  int32_t* count;                /* DEVICE int32 [B]: live entries per sequence */
  int32_t* seen;                 /* DEVICE int32 [B]: positions written so far */
  float gate_eps;                /* eps inside log(g + eps), >= 0 (1e-8 in the pages) */
  float gate_tau;                /* removal threshold, >= 0 (0.05 in the pages; 0 keeps all) */
  int32_t gate_sink;             /* leading positions never removed (4 in the pages) */
} sigattn_cache;

/* Build a cache from a prefill: the kept rows of k and v ([B][H][Lmax][d] bf16 described
 * by p: shapes, strides, seqlens; p->gate and p->gate_stride_b give the gates) are copied
 * to slots 0.. in position order, with their gates; count_b = number kept, seen_b = n_b.
 * The removal rule is the cache's (c->gate_tau, c->gate_sink); p's gate_tau, gate_sink
 * and gate_eps are not used. Requires p->dtype bf16, c->B == p->B, c->H == p->H,
 * c->d == p->d, c->cap >= every n_b, and c->gate != NULL exactly when p->gate != NULL. */
sigattn_status sigattn_cache_build(const sigattn_cache* c, const sigattn_problem* p,
                                   const void* k, const void* v, void* stream);

/* Write one new entry per sequence: k_new, v_new are DEVICE bf16 [B][H][d] with element
 * strides (stride_b, stride_h), rows 16-byte aligned; g_new is DEVICE float [B] (required
 * when the cache has gates, else must be NULL). The entry of sequence b, at position
 * seen_b, is kept iff the cache has no gates, gate_tau == 0, seen_b < gate_sink, or
 * g_new_b >= gate_tau; a kept entry goes to slot count_b. seen_b always advances. If a
 * kept entry finds its cache full (count_b == cap) it is not stored and, when status is
 * not NULL, the DEVICE int32 *status is set to 1 (it is never cleared by the library). */
sigattn_status sigattn_cache_append(const sigattn_cache* c, const void* k_new,
                                    const void* v_new, int64_t stride_b, int64_t stride_h,
                                    const float* g_new, int32_t* status, void* stream);

/* Bytes of device workspace sigattn_decode needs for this cache (the per-chunk partial
 * sums: B * H * ceil(cap / 512) * d floats), or -1 if the cache description is invalid. */
int64_t sigattn_decode_workspace_size(const sigattn_cache* c);

/* Single-query decode: o_bh = sum_{j < count_b} sigma(s q_bh . k_j + beta_b
 * [+ log(g_j + eps)]) [g_j] v_j (section 3 equation with the gate injection). q is DEVICE
 * bf16 [B][H][d] with element strides (stride_b, stride_h) (16-byte aligned rows); o has
 * the same strides, in out_dtype (SIGATTN_BF16 or SIGATTN_F32); count_b = 0 gives 0.
 * bias is a HOST float [B] array, required: beta_b, the bias the model uses for that
 * sequence (the pages' -log n). scale 0 selects 1/sqrt(d). workspace: DEVICE, at least
 * sigattn_decode_workspace_size(c) bytes, 16-byte aligned, owned by the caller; calls
 * that share a workspace must not overlap in time. Must not alias any other argument. */
sigattn_status sigattn_decode(const sigattn_cache* c, const void* q, int64_t stride_b,
                              int64_t stride_h, const float* bias, float scale, void* o,
                              int32_t out_dtype, void* workspace, int64_t workspace_bytes,
                              void* stream);

/* Single-query decode that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory or call hipMalloc (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same arguments, results and errors
 * as sigattn_decode without workspace and workspace_bytes; the per-chunk partial sums go
 * to a static device array inside the library instead, SIGATTN_NOALLOC_WORKSPACE_BYTES
 * (16 MiB) on every GPU the library runs on, held until the process ends. A cache whose
 * sigattn_decode_workspace_size exceeds that limit returns SIGATTN_ERR_UNSUPPORTED and
 * nothing is enqueued. Every call on one GPU shares that GPU's array and leaves the last
 * call's partial sums in it (each call writes the entries it reads before reading them):
 * calls that overlap in time on one GPU (different streams, or different host threads
 * without ordering) race and give undefined results. The first call on each device looks
 * up the array's device address (hipGetSymbolAddress); later calls reuse it. */
#define SIGATTN_NOALLOC_WORKSPACE_BYTES (16LL << 20)
sigattn_status sigattn_decode_noalloc(const sigattn_cache* c, const void* q, int64_t stride_b,
                                      int64_t stride_h, const float* bias, float scale, void* o,
                                      int32_t out_dtype, void* stream);

/* Host-side view of the work list a pass launches, for inspection and tests.
 * pass: 0 forward, 1 dq, 2 dk/dv, 3 the one-call backward of sigattn_bwd (d = 64 only),
 * whose dQ items are written as (b, h, -1 - tile). Writes up to `cap` items as
 * (b, h, tile) int32 triples into `items` (may be NULL when cap is 0) in launch order,
 * and the tile height in rows into *tile_rows (may be NULL). Returns the number of
 * compute items, or -1 if the problem is invalid. Fully padded tiles never appear.
 * Causal batches whose sequences all have one length are listed tile by tile (every
 * (sequence, head) of one tile together), costliest tiles first; in the one-call list
 * the dK/dV and dQ tiles are interleaved by cost. */
int64_t sigattn_plan(const sigattn_problem* p, int32_t pass, int32_t* items, int64_t cap,
                     int32_t* tile_rows);

/* Measurement aid (no attention work): the bf16 MFMA rate and shader clock this GPU
 * sustains, against which the attention kernels' throughput is also reported. Launches
 * nblocks workgroups of 256 threads on `stream`; every wave runs `iters` iterations of 16
 * v_mfma_f32_32x32x16_bf16 on four independent register accumulators, with no memory
 * traffic in the loop. sink: DEVICE float [nblocks * 256], 4-byte aligned, one value
 * per thread that keeps the products live (contents meaningless). clk: DEVICE int64
 * [2 * nblocks], 8-byte aligned: per workgroup, its elapsed shader-clock cycles
 * (s_memtime) and 100 MHz ticks (s_memrealtime); sum(cycles) / sum(ticks) * 100 is
 * the clock in MHz. Both buffers are owned by the caller and valid once the stream is
 * synchronised. 1 <= nblocks <= SIGATTN_MAX_CALIB_BLOCKS, 1 <= iters <=
 * SIGATTN_MAX_CALIB_ITERS and nblocks * iters <= SIGATTN_MAX_CALIB_WORK (a launch of at
 * most a few tens of milliseconds), else SIGATTN_ERR_INVALID_ARG; misaligned buffers
 * give SIGATTN_ERR_ALIGNMENT. Nothing is enqueued on error. */
#define SIGATTN_MAX_CALIB_BLOCKS (1 << 16)
#define SIGATTN_MAX_CALIB_ITERS (1 << 20)
#define SIGATTN_MAX_CALIB_WORK (1LL << 24)
sigattn_status sigattn_calibrate_mfma(int32_t nblocks, int32_t iters, float* sink,
                                      int64_t* clk, void* stream);
/* The matrix-core flops one sigattn_calibrate_mfma call performs (0 for invalid sizes). */
double sigattn_calibrate_mfma_flops(int32_t nblocks, int32_t iters);

const char* sigattn_status_string(sigattn_status s);
int sigattn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SIGATTN_H */
