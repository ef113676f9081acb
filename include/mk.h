/*
 * mk.h — C ABI of the multi-row speculative-verification decode step for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (from the pages):
 *   - richland.au, "Fusing the whole speculative-decoding cycle into one CUDA
 *     kernel", section "What shipped": one pass runs the main model over
 *     T = 1 + n_draft rows, then lm_head and verification on the device, and
 *     the host reads back only the accepted tokens; the Gated DeltaNet state is
 *     committed only through the surely-accepted token and drafts are replayed
 *     from a small (k, v, g, beta) ring; the GEMV shares activations so that
 *     T rows cost about the memory time of one.
 *   - richland.au, "OpenJet's CUDA megakernel runs 4 coding agents on one RTX
 *     3090", section "Why it matters": every step streams all weights once and
 *     multiplies each loaded weight against all stacked rows (4 agents x
 *     [token + 2 drafts] = 12 rows) while it is on chip.
 *   - pulse-3k2, "UPDATE: ... KL divergence 0.0009 vs llama.cpp", section
 *     "Decode accuracy": greedy output is exactly the main model's greedy choice.
 * The block format (Q4_K-style: 256-weight superblocks with fp16 d and dmin,
 * eight 32-weight sub-blocks with 6-bit scale sc and min m, 4-bit codes q,
 * w = d*sc*q - dmin*m) and the per-32 int8 activation quantization follow the
 * workload definition that accompanies those pages.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the name starts with h_ (host).
 *     Arrays are row-major and contiguous.  The caller owns every buffer; the
 *     library never allocates or frees device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous on that stream unless stated otherwise.
 *   - Arguments are validated on the host first.  On error the call returns a
 *     negative MK_ERR_* code, enqueues nothing and records a message that
 *     mk_last_error() returns (thread-local).  No call prints or aborts.
 *   - Alignment: Q4K blobs 256 B, every other buffer 16 B (MK_ERR_ALIGN).
 *   - Row counts T are 1..16 (MK_T_MAX), and 1..24 for mk_decode_step
 *     (MK_STEP_T_MAX) (MK_ERR_RANGE).  Reduction orders are fixed, so
 *     a call is bit-reproducible for the same inputs and the same T.
 *   - Concurrent calls on different streams need distinct workspaces.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MK_OK = 0,
  MK_ERR_ARG = -1,       /* NULL pointer or invalid enum value            */
  MK_ERR_SHAPE = -2,     /* dimension not allowed (e.g. n_in % 256 != 0)  */
  MK_ERR_ALIGN = -3,     /* misaligned pointer                            */
  MK_ERR_RANGE = -4,     /* value outside its documented range            */
  MK_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required       */
  MK_ERR_LAUNCH = -6,    /* a HIP launch or copy failed                   */
  MK_ERR_COOP = -7,      /* cooperative launch not possible on the device */
  MK_ERR_DEVICE = -8     /* no usable device, or a device-side error word */
};

#define MK_T_MAX 16
#define MK_STEP_T_MAX 24 /* rows of one decode step: up to 8 agents x 3 rows */
/* Largest KV cache capacity (positions per agent and KV head) of the
 * attention calls: the kernels address a head's cache with 32-bit byte offsets. */
#define MK_ATTN_CAP_MAX (1 << 26)

const char* mk_status_string(int status);
const char* mk_last_error(void);
int mk_version(void);

/* Binds the calling thread's current device and queries its CU count and
 * co-residency limits.  Idempotent.  Returns MK_ERR_DEVICE without a GPU. */
int mk_init(int device);

/* ------------------------------------------------------------------ weights */
/* A Q4_K-style matrix of n_out x n_in weights in the library's device layout
 * (see mk_q4k_pack).  n_in % 256 == 0.  `blocks` is 256-B aligned. */
typedef struct {
  const void* blocks;
  int32_t n_out, n_in;
} mk_q4k;

/* Bytes of the packed layout: 144 B per 256 weights, rows padded to a
 * multiple of 64 (padding rows are zero and never written to outputs). */
size_t mk_q4k_bytes(int32_t n_out, int32_t n_in);

/* Host-side conversion between field arrays and the packed layout.
 * Fields (as produced by a generator or a model loader):
 *   h_d, h_dmin [n_out][n_in/256]   fp16 bit patterns
 *   h_sc, h_m   [n_out][n_in/256][8] values 0..63
 *   h_q         [n_out][n_in]        values 0..15
 * Packed layout: 64-row tiles; each (tile, superblock) unit is 9216 B = a
 * 1024-B header block (row r: d, dmin, 12 B of scales) and eight 1024-B code
 * blocks (sub-block j, row r: 16 B holding 32 codes).  Pack rows [r0, r1)
 * only (r0 % 64 == 0) so large matrices can be packed in slices; h_blocks then
 * points at the unit of tile r0/64.  Returns MK_ERR_RANGE for a field value
 * outside its range. */
int mk_q4k_pack(const uint16_t* h_d, const uint16_t* h_dmin, const uint8_t* h_sc, const uint8_t* h_m,
                const uint8_t* h_q, int32_t n_out, int32_t n_in, int32_t r0, int32_t r1, void* h_blocks);
int mk_q4k_unpack(const void* h_blocks, int32_t n_out, int32_t n_in, uint16_t* h_d, uint16_t* h_dmin,
                  uint8_t* h_sc, uint8_t* h_m, uint8_t* h_q);

/* ------------------------------------------------------ activation quantizer */
/* Per row t and group of 32 consecutive elements: s = amax/127 (IEEE fp32
 * division, amax over the group's non-NaN elements), a8 = clamp(rne(x/s),
 * -127, 127), gsum = sum of a8.  When s is 0 (an all-zero group, or amax at
 * most 63 * 2^-149 so that amax/127 underflows) or the group is all NaN, s = 0
 * and every code is 0; an element whose x/s is NaN codes as 0.  x [T][K], a8 [T][K], s and gsum [T][K/32]; K % 32 == 0.
 * Bit-identical to the CPU definition. */
int mk_quantize_rows(const float* x, int32_t T, int32_t K, int8_t* a8, float* s, int32_t* gsum, void* stream);

/* ----------------------------------------------------------------- T-row GEMV */
/* richland.au, "Fusing the whole speculative-decoding cycle into one CUDA
 * kernel", section "What shipped" (the GEMV shares its activations so that T
 * rows cost about the memory time of one), and the 4-agent article, section
 * "Why it matters" (each loaded weight is multiplied against every stacked row
 * while it is on chip).
 * y[t][o] = sum_k w[o][k] * s[t][k/32] * a8[t][k] for the quantized rows of x:
 * every weight block is read from HBM once and multiplied against all T rows.
 * Integer sub-block sums (32 codes x 32 int8 values) are exact; they are
 * combined with d, dmin, sc, m and the activation scales in fp32.
 * x [T][n_in] fp32, y [T][n_out] fp32.  Workspace from mk_qgemv_rows_workspace. */
size_t mk_qgemv_rows_workspace(int32_t T, int32_t n_out, int32_t n_in);
int mk_qgemv_rows(const mk_q4k* W, const float* x, int32_t T, float* y, void* ws, size_t ws_bytes, void* stream);

/* Same, with the inner-product engine chosen explicitly:
 * MK_PATH_AUTO (MK_PATH_DOT4 for T <= 4, MK_PATH_STEP from T = 5: the
 * faster one on the 5120 x 5120 workload), MK_PATH_DOT4 (packed int8 dot
 * products, T <= 8) or MK_PATH_MFMA (int8 matrix cores, rows padded to 16);
 * those two give bit-identical results.
 * MK_PATH_STEP streams the matrix through the decode step's own engines and
 * activation records: the records are written by the step's epilogue
 * quantizer (the rule of mk_quantize_rows) and each 64-row unit goes through
 * the engine the step uses for T rows (dot4 at T = 1; two sub-blocks per
 * 16x16x64 int8 matrix product up to 8 padded rows; one sub-block per
 * 16x16x32 product above), loaded by LDS-DMA two units ahead of the
 * arithmetic, one block of 4 streaming waves per CU (a block's waves hand
 * their sums over through LDS with bounded waits; blocks never wait for
 * each other).  Its results equal the
 * other paths' up to the order of the fp32 sums, and the step's engines can
 * be checked through it outside the persistent launch.  The workspace then
 * begins with the records, one per superblock b of x (5120 B): codes
 * [sub-block j][octet q][row t < 16][8 B] (the 8 codes of elements
 * 256 b + 32 j + 8 q .. + 7; rows >= T zero), then s [j][t] and s * gsum
 * [j][t] as fp32 ([8][16] each).
 * Launches: the activation quantizer (which also clears the tile counters in
 * the workspace), then the GEMV, whose last block per 64-row tile adds the
 * tile's split-K partials in a fixed order; no memset, so the call can be
 * captured in a HIP graph.  Calls that share a workspace must not overlap. */
enum { MK_PATH_AUTO = 0, MK_PATH_DOT4 = 1, MK_PATH_MFMA = 2, MK_PATH_STEP = 3 };
int mk_qgemv_rows_ex(const mk_q4k* W, const float* x, int32_t T, float* y, int32_t path, void* ws,
                     size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * T-row GEMV as mk_qgemv_rows_ex (same engines, bit-identical results), with
 * its workspace in a static device array of MK_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that each GPU the library runs on holds until the process ends.
 * A call whose workspace (mk_qgemv_rows_workspace) would exceed the array
 * returns MK_ERR_WORKSPACE and enqueues nothing; every shape of the 27B-class
 * stack fits at any T.  Allocates nothing: no hipMalloc or hipFree, no
 * allocating library call.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents (the launches clear the counters that
 * must start at zero themselves, without a memset): calls that overlap on one
 * GPU (several streams or threads) race. */
#define MK_NOALLOC_SCRATCH_BYTES (16u << 20)
int mk_qgemv_rows_noalloc(const mk_q4k* W, const float* x, int32_t T, float* y, int32_t path, void* stream);

/* ------------------------------------------------------------------ FFN block */
/* y = W_down . q8(SiLU(W_gate . q8(x)) * (W_up . q8(x))); gate, up are
 * F x H, down is H x F.  x, y [T][H] fp32; h_out (optional, NULL to skip)
 * receives the fp32 intermediate [T][F].  Three launches: quantizer, gate/up
 * (whose tile epilogues apply SiLU(g) * u and quantize h), down; from T = 4
 * on the engines of MK_PATH_STEP, below on those of MK_PATH_DOT4 (the faster
 * ones on the 5120 -> 17408 -> 5120 workload). */
size_t mk_ffn_rows_workspace(int32_t T, int32_t H, int32_t F);
int mk_ffn_rows(const mk_q4k* gate, const mk_q4k* up, const mk_q4k* down, const float* x, int32_t T, float* y,
                float* h_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- lm_head + verify */
/* richland.au single-stream article, section "What shipped" (lm_head and
 * verification run on the device; only accepted tokens go back to the host),
 * and pulse-3k2 "UPDATE: ... KL divergence 0.0009 vs llama.cpp", section
 * "Decode accuracy vs llama.cpp" (greedy output equals the main model's greedy
 * choice).
 * logits[t][v] = sum_h f32(W[v][h]) * hid[t][h] (fp16 weights widened exactly,
 * fp32 hidden, fp32 accumulation); argmax[t] = lowest index of the maximum
 * (NaN never wins; -1 if all logits of the row are NaN).  Rows are split into
 * G groups by h_group_start[0..G] (host array, h_group_start[0] = 0,
 * h_group_start[G] = T, every group non-empty; NULL = one group of T rows).
 * Group g has n = rows and n-1 drafts at drafts[h_group_start[g] - g ...];
 * draft i is accepted when it equals argmax of the group's row i.  n_acc[g] =
 * number of leading accepted drafts; tokens[h_group_start[g] + i] for
 * i = 0..n_acc[g] receives the accepted drafts then the argmax of row n_acc[g]
 * (other slots are set to -1).  A draft id outside [0, V) is a mismatch.
 * W [V][H] fp16 bits, hid [T][H], drafts [T-G] int32 (may be NULL if T == G),
 * argmax [T], n_acc [G], tokens [T] (all device).  H % 64 == 0.
 * Range of hid: any fp32 values.  Each row is multiplied by an exact power of
 * two that brings its largest magnitude into [2^14, 2^15) before it is split
 * into the two fp16 parts the matrix cores take, so neither part overflows and
 * every element within 2^-24 of the row's largest keeps about 22 bits; the
 * scaling multiplies every logit of a row by the same power of two and leaves
 * the argmax unchanged.  A row holding inf is not scaled. */
size_t mk_lmhead_verify_workspace(int32_t V, int32_t H, int32_t T);
int mk_lmhead_verify(const uint16_t* W_f16, int32_t V, int32_t H, const float* hid, int32_t T,
                     const int32_t* h_group_start, int32_t G, const int32_t* drafts, int32_t* argmax,
                     int32_t* n_acc, int32_t* tokens, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------- sampling-mode verification */
/* pulse-3k2, "UPDATE: ... KL divergence 0.0009 vs llama.cpp", section
 * "Decode accuracy vs llama.cpp": with sampling, speculative decoding keeps
 * the same distribution as without drafts; top_k is capped at 32
 * (richland.au single-stream article, "Caveats"; 4-agent article, limits).
 * The pages give no acceptance rule; this is speculative sampling with each
 * draft a deterministic proposal.  Logits as in mk_lmhead_verify.  Row t's
 * target p_t is the softmax of its top_k largest logits (NaN never counts,
 * ties go to the lower index) divided by `temperature`.  Groups and drafts
 * as in mk_lmhead_verify.  In group g, draft i is accepted when
 * u_acc[row i] < p_i(draft i) (0 for a token outside the top_k); at the first
 * rejection, row i emits a sample of p_i with the draft removed, picked by
 * u_samp[row i] through the inverse CDF over the candidates in ascending
 * vocabulary order; if every draft is accepted, the last row emits a sample
 * of its p (u_samp).  Every emitted token is then distributed exactly as the
 * row's p.  A row whose logits are all NaN has no candidate: it rejects its
 * draft and emits -1.
 *   u_acc, u_samp [T] fp32 in [0, 1) (device): the caller's uniform numbers
 *   topk_idx [T][32] int32, topk_logit [T][32] fp32 (device, optional, NULL
 *     to skip): each row's candidates in ascending vocabulary order, unused
 *     slots -1 / -inf
 *   n_acc [G], tokens [T] (device) as in mk_lmhead_verify.
 * 1 <= top_k <= 32 and 0 < temperature < inf (MK_ERR_RANGE otherwise);
 * H % 64 == 0; V <= 2^21 (MK_ERR_SHAPE).  Six launches: the rows' prescale
 * exponents, the lm_head fragments, the lm_head stream writing every logit
 * into the workspace, the top-k of every 8192-logit chunk (staged in LDS),
 * the top-k of every row from its chunks' candidates, the accept / resample
 * pass.
 * The hidden rows are prescaled as in mk_lmhead_verify; the logits returned
 * in topk_logit are scaled back exactly. */
size_t mk_lmhead_sample_workspace(int32_t V, int32_t H, int32_t T);
int mk_lmhead_sample(const uint16_t* W_f16, int32_t V, int32_t H, const float* hid, int32_t T,
                     const int32_t* h_group_start, int32_t G, const int32_t* drafts, int32_t top_k, float temperature,
                     const float* u_acc, const float* u_samp, int32_t* topk_idx, float* topk_logit, int32_t* n_acc,
                     int32_t* tokens, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- MTP draft loop */
/* richland.au single-stream article, section "What shipped": after the
 * verification, MTP catch-up rows for the accepted tokens, then n_draft MTP
 * draft steps, with drafting restricted to the 32,768 most frequent tokens;
 * the 4-agent article, section "Why it matters": every agent drafts its own
 * tokens in the same rows.  The pages name the head's work, not its layers;
 * the synthetic head here is one pass of
 *   z = [RMSNorm(f32 E[token]) ; RMSNorm(hidden)],  u = fc . q8(z),
 *   x' = u + FFN(RMSNorm(u))   (FFN as in the stack),
 * with the embedding E tied to the lm_head.  A draft is the argmax of
 * RMSNorm(x') over the first V_draft rows of E (lowest index on ties, NaN never
 * wins).
 * Pass 0 (catch-up) runs every row t of the step: group g's rows
 * i = 0..n_acc[g] pair the main model's final residual hidden[gs[g] + i] with
 * the token emitted after it, tokens[gs[g] + i] (the accepted drafts, then
 * the bonus token, as mk_lmhead_verify writes them); row gs[g] + n_acc[g]
 * gives group g's draft 1.  Pass k = 1..n_draft-1 runs one row per group:
 * draft k with the x' of the row that produced it gives draft k + 1.  Every
 * pass reads the head's weights once for all of its rows; n_acc and the
 * drafts are read on the device, so the loop never returns to the host.
 *   m: fc is H x 2H (H % 256 == 0); gate, up F x H; down H x F
 *   embed_f16 [V][H] fp16 bits (device), V_draft <= V
 *   hidden [T][H] fp32, tokens [T] int32, n_acc [G] int32 (device)
 *   drafts [n_draft][G] int32 (device output); a group whose n_acc is outside
 *     0..rows-1 gets -1 for every draft
 *   trace (device, optional): [T + G (n_draft - 1)][H] x' of every row of
 *     every pass (pass 0's rows past a group's n_acc are not catch-up rows:
 *     they run on zero inputs and their values carry no meaning)
 * 1 <= T <= 16, groups as in mk_lmhead_verify, 1 <= n_draft <= 16.
 * Asynchronous on `stream` (several launches per pass). */
typedef struct {
  mk_q4k fc, gate, up, down;
} mk_mtp;
size_t mk_mtp_draft_workspace(const mk_mtp* m, int32_t V_draft, int32_t T, int32_t G);
int mk_mtp_draft(const mk_mtp* m, const uint16_t* embed_f16, int32_t V, int32_t V_draft, const float* hidden,
                 int32_t T, const int32_t* h_group_start, int32_t G, const int32_t* tokens, const int32_t* n_acc,
                 int32_t n_draft, int32_t* drafts, float* trace, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- Gated DeltaNet */
/* richland.au single-stream article, section "What shipped": the recurrent
 * state is committed only through the surely-accepted token, and drafted rows
 * are replayed from a small (k, v, g, beta) ring.  The delta rule itself
 * (S <- g (I - beta k k^T) S + beta k v^T, o = S^T q) follows the workload
 * definition that accompanies the pages.
 * State of nh independent heads (e.g. layers x heads) with rollback ring.
 *   S     [nh][dk][dv] fp32, S[h][i][j] (i key index, j value index)
 *   ring  [2][nh][T_max-1][dk+dv+2] fp32: two halves used on alternate steps;
 *         a step stores its rows 1..T-1 as (k, v, g, beta) in one half while
 *         it replays the previous step's rows from the other half
 *   n_acc 4 int32 (device): [0] accept length of the last step, read by the
 *         next step to replay ring rows 1..n_acc[0] (the decode step writes
 *         it from its verification); [1] the half holding the last step's rows;
 *         [2] status word: set to 1 by a step or commit that read an accept
 *         length outside 0..T_max-1 (it then replays nothing);
 *         [3] unused.  Zero-initialise all four before the first step.
 * dk = dv = 128 (the only head size supported).  2 <= T_max <= 16. */
typedef struct {
  float* S;
  float* ring;
  int32_t* n_acc;
  int32_t nh, dk, dv, T_max;
} mk_deltanet;

/* One step, per head: replay ring rows 1..a (a = n_acc[0] if use_prev_acc,
 * else 0; a value outside 0..T_max-1 replays nothing and sets n_acc[2], which
 * mk_deltanet_status reports), then for t = 0..T-1:
 *   S <- g_t (I - beta_t k_t k_t^T) S + beta_t k_t v_t^T,   o_t = S^T q_t,
 * committing S after row 0 and storing rows 1..T-1 in the ring.
 * q, k [T][nh][dk]; v [T][nh][dv]; g, beta [T][nh]; o [T][nh][dv].  1 <= T <= T_max. */
int mk_deltanet_step(const mk_deltanet* st, int32_t use_prev_acc, const float* q, const float* k, const float* v,
                     const float* g, const float* beta, int32_t T, float* o, void* stream);

/* Replays ring rows 1..a (a = n_acc[0]; outside 0..T_max-1: nothing, and
 * n_acc[2] is set) into S without new rows, so that S holds the state through
 * the accepted row; then sets n_acc[0] = 0. */
int mk_deltanet_commit(const mk_deltanet* st, void* stream);

/* Synchronises `stream`, reads the status word n_acc[2] and clears it.
 * Returns MK_ERR_RANGE if a step or commit since the last call read an accept
 * length outside 0..T_max-1, else MK_OK. */
int mk_deltanet_status(const mk_deltanet* st, void* stream);

/* --------------------------------------------------- persistent decode step */
/* richland.au single-stream article, section "What shipped" (one persistent
 * launch runs the main model over T = 1 + n_draft rows, lm_head and the
 * verification; the host reads back only the accepted tokens), and the
 * 4-agent article, section "Why it matters" (all agents' rows share one
 * weight read per step).
 * A synthetic layer stack: per layer a = RMSNorm(x); x += P_out.q8(P_in.q8(a));
 * a = RMSNorm(x); x += W_down.q8(SiLU(W_gate.q8(a)) * W_up.q8(a)).  RMSNorm has
 * unit gain and eps 1e-6; the norm scale is applied to the activation scales
 * (equal in exact arithmetic to quantizing the normalised row).  Layers with
 * gdn_layer[l] != 0 also run one Gated DeltaNet step per agent in their mixer
 * slot on the caller's seeded inputs (its output is not fed back).  After the
 * last layer: final RMSNorm, lm_head, argmax and verification per group. */
typedef struct {
  int32_t n_layers, hidden, proj, ffn, vocab;
  const mk_q4k* p_in;  /* [n_layers], proj x hidden   */
  const mk_q4k* p_out; /* [n_layers], hidden x proj   */
  const mk_q4k* gate;  /* [n_layers], ffn x hidden    */
  const mk_q4k* up;    /* [n_layers], ffn x hidden    */
  const mk_q4k* down;  /* [n_layers], hidden x ffn    */
  const uint16_t* lm_head; /* [vocab][hidden] fp16 bits */
  const uint8_t* h_gdn_layer; /* host [n_layers] flags, NULL = none */
  int32_t n_agents;           /* Gated DeltaNet states (one per verify group) */
  const mk_deltanet* dn;      /* host array [n_agents]; nh = gdn layers * heads */
} mk_stack_desc;

typedef struct mk_stack mk_stack; /* opaque host-side descriptor */
int mk_stack_create(const mk_stack_desc* desc, mk_stack** out);
void mk_stack_destroy(mk_stack* st);
size_t mk_decode_step_workspace(const mk_stack* st, int32_t T);

/* One decode step in ONE persistent launch, then one D->H copy of the
 * emitted tokens and accept lengths and one stream synchronisation.
 * 1 <= T <= MK_STEP_T_MAX (24: the 4-agent article, section "Caveats",
 * allows up to 8 agents, 3 rows each); above 16 rows every weight is still
 * read once, and the lm_head is streamed once per 16 rows.
 *   x [T][hidden] (in: step input rows; out: final residual),
 *   h_group_start as in mk_lmhead_verify (G groups == agents when GDN is on),
 *   drafts [T-G] (device), gdn_* [T][nh][d] (device seeded inputs, NULL when
 *   the stack has no GDN layers), gdn_o [T][nh][dv] (device, may be NULL),
 *   h_tokens [T], h_n_acc [G] (host outputs), d_argmax [T] (device, optional),
 *   trace (device, optional): [n_layers][T][hidden] residual after each layer.
 * The workspace holds the stack's weight table and work plans: it is bound
 * to the last stack that ran a step on it.  A step by another stack uploads
 * its own tables first (host-side record per workspace).  If some other call
 * wrote the workspace in between, the kernel sees a foreign tag, nothing
 * runs, and the call returns MK_ERR_WORKSPACE; the next call uploads the
 * tables again.  Steps that share a workspace, or a stack, must not overlap
 * (a stack also holds the pinned host buffer its steps read back into and
 * the events around its last launch).
 * The lm_head input rows are RMSNorm outputs, so |value| <= sqrt(hidden); they
 * are multiplied by the exact power of two 2^k with sqrt(hidden) 2^k <= 2^14
 * before the fp16 split (the argmax is unchanged).
 * Returns MK_ERR_DEVICE if a bounded device wait ran out (watchdog), and
 * MK_ERR_RANGE if an agent state's accept length was outside 0..T_max-1
 * (that agent then replays nothing; its n_acc[2] is set as well). */
int mk_decode_step(mk_stack* st, float* x, int32_t T, const int32_t* h_group_start, int32_t G,
                   const int32_t* drafts, const float* gdn_q, const float* gdn_k, const float* gdn_v,
                   const float* gdn_g, const float* gdn_beta, float* gdn_o, int32_t* h_tokens, int32_t* h_n_acc,
                   int32_t* d_argmax, float* trace, void* ws, size_t ws_bytes, void* stream);

/* The same step with the full-attention layers' attention in the persistent
 * launch (richland.au single-stream article, "What shipped": 16 full gated
 * attention layers beside 48 Gated DeltaNet layers, decoded by split-K flash
 * decoding; the 4-agent article, "Why it matters": what grows with the
 * agents is attention, each agent reading its own KV cache).  Like the
 * Gated DeltaNet steps, the attention runs on the caller's seeded inputs
 * beside the layer pipeline (its output is not fed back), so that its
 * reads and time are part of the step.  For each of n_layers layers and each
 * agent g (the verify groups of h_group_start), the result is that of
 * mk_attn_decode on that layer's q, gate and caches:
 *   q, gate, o   [n_layers][T][Hq][128] fp32 (gate may be NULL)
 *   h_ctx        host [G]: positions cached before this step's rows; the
 *                agent's n_g new rows are at h_ctx[g] .. h_ctx[g] + n_g - 1
 * and either an fp16 cache (the q8_0 pointers NULL):
 *   k_cache      [n_layers][G][Hkv][cap][128] fp16 bits, position-major
 *   v_cache      [n_layers][G][Hkv][128][cap] fp16 bits, dimension-major
 * or a q8_0 cache (k_cache and v_cache NULL; the layouts of
 * mk_attn_decode_q8 with a leading layer dimension; the result is that of
 * mk_attn_decode_q8):
 *   k_codes [n_layers][G][Hkv][cap][128] int8, k_scales [n_layers][G][Hkv][cap][4],
 *   v_codes [n_layers][G][Hkv][cap/64][128][64] int8, v_scales [n_layers][G][Hkv][cap/32][128]
 * All device, 16-B aligned.  cap % 64 == 0, cap <= MK_ATTN_CAP_MAX,
 * h_ctx[g] + n_g <= cap, n_g * Hq/Hkv <= 16 (MK_ERR_SHAPE / MK_ERR_RANGE
 * otherwise); neither or both cache formats given is MK_ERR_ARG.
 * attn == NULL is mk_decode_step.  The workspace
 * (mk_decode_step_attn_workspace) adds the split partials to the step's. */
typedef struct {
  int32_t n_layers, Hq, Hkv, cap;
  const int32_t* h_ctx;
  const float* q;
  const float* gate;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  float* o;
  const int8_t* k_codes;
  const uint16_t* k_scales;
  const int8_t* v_codes;
  const uint16_t* v_scales;
} mk_step_attn;
size_t mk_decode_step_attn_workspace(const mk_stack* st, int32_t T, const int32_t* h_group_start, int32_t G,
                                     const mk_step_attn* attn);
int mk_decode_step_attn(mk_stack* st, float* x, int32_t T, const int32_t* h_group_start, int32_t G,
                        const int32_t* drafts, const float* gdn_q, const float* gdn_k, const float* gdn_v,
                        const float* gdn_g, const float* gdn_beta, float* gdn_o, int32_t* h_tokens, int32_t* h_n_acc,
                        int32_t* d_argmax, float* trace, const mk_step_attn* attn, void* ws, size_t ws_bytes,
                        void* stream);

/* Duration in ms of the last mk_decode_step's persistent launch on this
 * stack, from HIP events recorded around the launch on its stream (-1 if
 * unavailable). */
float mk_decode_step_last_ms(const mk_stack* st);

/* Profiling aid: copies (synchronously) the device clock stamps the last
 * mk_decode_step on workspace `ws` recorded: stamp 0 at the launch start,
 * stamp i after the i-th grid barrier (1 + 4 per layer + 1 of them), and the
 * last of the n_max at the launch end.  h_clock_hz receives the clock rate.
 * Returns the number of stamps copied or a negative status. */
int mk_decode_step_stamps(const mk_stack* st, int32_t T, const void* ws, uint64_t* h_stamps, int32_t n_max,
                          int64_t* h_clock_hz);

/* ------------------------------------------------------- full attention */
/* Decode-time attention of the full-attention layers over an fp16 KV cache,
 * by split-K flash decoding (richland.au, "Fusing the whole speculative-
 * decoding cycle into one CUDA kernel", section "What shipped").  Rows are
 * split into G agents by h_group_start as in mk_lmhead_verify; agent g has
 * h_ctx[g] positions cached before this step, and its n_g new rows (token +
 * drafts) have their k, v already stored at positions h_ctx[g] ..
 * h_ctx[g] + n_g - 1.  Row i of agent g sees positions 0 .. h_ctx[g] + i
 * (causal among the drafts).  For query head hq and its KV head
 * h = hq / (Hq / Hkv):
 *   o[t][hq] = sum_j softmax_j(q[t][hq] . K[g][h][j] / sqrt(d)) V[g][h][.][j],
 * then o *= 1 / (1 + exp(-gate)) elementwise when gate is not NULL (the
 * output gate of gated attention).
 *   q, gate, o  [T][Hq][d] fp32 (device; gate may be NULL)
 *   k_cache     [G][Hkv][cap][d] fp16 bits (device), position-major
 *   v_cache     [G][Hkv][d][cap] fp16 bits (device), dimension-major
 *   h_ctx [G], h_group_start [G+1] (host; NULL = one group of T rows)
 * d = 128; cap % 64 == 0; cap <= MK_ATTN_CAP_MAX; h_ctx[g] + n_g <= cap; n_g * Hq/Hkv <= 64;
 * G <= 16.  Slots past an agent's last position are never used (they may
 * hold anything).  Two launches (split pass, merge + gate); the workspace
 * size depends on the contexts and the device (mk_attn_decode_workspace).
 * fp32 accumulation; the products carry about 22 bits (q and the softmax
 * weights are split into two fp16 parts). */
size_t mk_attn_decode_workspace(int32_t T, int32_t Hq, int32_t Hkv, const int32_t* h_ctx,
                                const int32_t* h_group_start, int32_t G);
int mk_attn_decode(const float* q, const float* gate, int32_t T, int32_t Hq, const uint16_t* k_cache,
                   const uint16_t* v_cache, int32_t Hkv, int32_t d, int32_t cap, const int32_t* h_ctx,
                   const int32_t* h_group_start, int32_t G, float* o, void* ws, size_t ws_bytes, void* stream);

/* The same attention over a q8_0 KV cache (the pages switch the cache to
 * q8_0 above about 80K positions; same page and section).  A q8_0 block is
 * 32 int8 codes with one fp16 scale; a value is f32(scale) * code.
 *   k_codes  [G][Hkv][cap][d] int8, position-major
 *   k_scales [G][Hkv][cap][d/32] fp16 bits: scale of dims 32i..32i+31 of a position
 *   v_codes  [G][Hkv][cap/64][d][64] int8, tile-major: positions 64t..64t+63
 *            of every dimension together, so that one 64-position tile of a
 *            head is one contiguous run
 *   v_scales [G][Hkv][cap/32][d] fp16 bits: scale of positions 32i..32i+31 of a dimension
 * All device, 16-B aligned.  Every other argument, the workspace (the same
 * mk_attn_decode_workspace) and the errors are those of mk_attn_decode.
 * Scales of blocks that hold no visible position are never used. */
int mk_attn_decode_q8(const float* q, const float* gate, int32_t T, int32_t Hq, const int8_t* k_codes,
                      const uint16_t* k_scales, const int8_t* v_codes, const uint16_t* v_scales, int32_t Hkv,
                      int32_t d, int32_t cap, const int32_t* h_ctx, const int32_t* h_group_start, int32_t G,
                      float* o, void* ws, size_t ws_bytes, void* stream);

/* Measurement aid, not a step of the method: reads `bytes` bytes of buf
 * (device, 16-B aligned, bytes % 16 == 0) once with 16-B nontemporal loads
 * spread over the whole device, and may write one word to *sink (device, 4-B
 * aligned) so that the loads cannot be dropped.  The time of a call over a
 * buffer far larger than the caches is the read bandwidth the device
 * attains, reported beside the 8 TB/s peak.  Asynchronous on `stream`. */
int mk_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
