// mk_internal.h — host-side launchers shared between the C-ABI layer and the
// kernel translation units of libmk.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

// Records a thread-local error message for mk_last_error() and returns status.
int set_error(int status, const char* fmt, ...);

constexpr int kTPadHost = 16;         // activation-scale rows padded to 16
constexpr int kUnitBytesHost = 9216;  // 64 rows x 144 B per superblock
constexpr int kDot4MaxT = 8;          // dot4 engine instances exist for T = 1..8
constexpr int kDot4MaxTAuto = 4;      // automatic choice: dot4 up to 4 rows, the streaming engines from 5
constexpr int kFfnStreamMinT = 4;     // mk_ffn_rows: dot4 launches below 4 rows, the streaming engines from 4

struct QActBuf {
  int8_t* a8;    // [T][K]
  float2* ssg;   // [K/32][16]
  int32_t K, T;
};

// x [T][K] -> a8/s/gsum (API arrays, each may be null) and/or the internal
// record (ssg may be null).  Zero-fills ssg rows T..15, and zero[0..nzero)
// (the tile counters of the GEMV launches that follow on the stream).
hipError_t launch_quantize(const float* x, int T, int K, int8_t* a8, float* s, int32_t* gsum, float2* ssg,
                           unsigned* zero, int nzero, hipStream_t st);

struct GemvPlan {
  int ntiles, nsb, per_wg, ksplit, nmat;
  size_t partial_elems;  // nmat * ksplit * T * ntiles*64
};
// The streaming GEMV and FFN on the step's engines and records (T <= 16);
// cu: the device's compute units (one block per CU).
size_t engine_gemv_workspace(int T, int N, int K, int cu);
hipError_t launch_engine_gemv(const uint8_t* W, int N, int K, const float* x, int T, float* y, uint8_t* ws, int cu,
                              hipStream_t st);
size_t engine_ffn_workspace(int T, int H, int F, int cu);
hipError_t launch_engine_ffn(const uint8_t* gate, const uint8_t* up, const uint8_t* down, int H, int F, const float* x,
                             int T, float* y, float* h_out, uint8_t* ws, int cu, hipStream_t st);

GemvPlan plan_gemv(int T, int n_out, int n_in, int nmat, int cu_count);

// What the last block of each tile does with the summed split-K partials.
enum { kEpiStore = 0, kEpiSiluQ8 = 1 };
struct GemvEpi {
  unsigned* tickets;  // [ntiles], zero when the GEMV starts (launch_quantize clears them)
  int kind;           // kEpiStore: y[t][o] = sum_ks partial[0][ks][t][o], o < n_out
                      // kEpiSiluQ8: h = SiLU(sum partial[0]) * sum partial[1], written to y if
                      //   not null and quantized into h8 / hssg (the next GEMV's activation rows)
  int n_out;
  float* y;
  int8_t* h8;
  float2* hssg;
};

// Writes partial[mat][ks][t][tile*64 + r] for both matrices of W (nmat 1 or
// 2) and runs the epilogue of each tile in the block that completes it.
hipError_t launch_gemv(const uint8_t* const* W, const GemvPlan& p, const QActBuf& act, int path, float* partial,
                       const GemvEpi& epi, hipStream_t st);

}  // namespace mk

#define MK_LM_MAX_G 16
namespace mk {
size_t lm_workspace_bytes(int V, int H);
hipError_t launch_lmhead(const uint16_t* W, int V, int H, const float* hid, int T, const int32_t* gs, int G,
                         const int32_t* drafts, int32_t* argmax, int32_t* n_acc, int32_t* tokens, void* ws,
                         int cu_count, hipStream_t st);
hipError_t launch_lm_stream(const uint16_t* W, int V, int H, const float* hid, int T, const int32_t* gs, int G,
                            const int32_t* drafts, int32_t* argmax, int32_t* n_acc, int32_t* tokens, void* ws,
                            int cu_count, hipStream_t st, float* logits, int* row_exp);

// Sampling-mode verification (mk_sample.hip): top-k of each row's logits,
// then the speculative-sampling accept/resample pass.
constexpr int kTopKMax = 32;
struct SampleArgs {
  const float* logits;   // [T][V], row t scaled by 2^row_exp[t]
  const int* row_exp;    // [16]
  int V, T, k;
  int32_t* cand_idx;     // [T][32], ascending vocabulary index, -1 past the row's candidates
  float* cand_val;       // [T][32], the logits (unscaled), -inf past the candidates
  int G;
  int gs[MK_LM_MAX_G + 1];
  const int32_t* drafts;
  float temperature;
  const float* u_acc;    // [T]
  const float* u_samp;   // [T]
  int32_t* n_acc;        // [G]
  int32_t* tokens;       // [T]
};
// part: the first level's candidates, sample_part_bytes(V, T) bytes.
constexpr int kSampleMaxVocab = 1 << 21;  // the second level's candidates fit its LDS up to this vocabulary
size_t sample_part_bytes(int V, int T);
hipError_t launch_sample(const SampleArgs& a, void* part, hipStream_t st);

// MTP draft loop (mk_mtp.hip): the row kernels around the GEMV, FFN and
// lm_head launches of each pass.
struct MtpArgs {
  const uint16_t* embed;  // [V][H] fp16 bits (the tied lm_head)
  int V, H, T, G;
  int gs[MK_LM_MAX_G + 1];
  const float* hidden;    // [T][H] main-model final residual
  const int32_t* tokens;  // [T] emitted tokens of the step
  const int32_t* n_acc;   // [G]
  int32_t* drafts;        // [n_draft][G]
  float* z;               // [T][2H] pass input
  float* u;               // [T][H] fc output
  float* y;               // [T][H] FFN output
  float* xp;              // [T][H] x' = u + y
  float* prev;            // [G][H] x' of the row that continues each group's chain
  float* hid;             // [G][H] RMSNorm(prev): the lm_head input
  int32_t* dead;          // [G] groups whose accept length was out of range
  float* trace;           // optional [T + G (n_draft - 1)][H]
};
hipError_t launch_mtp_in(const MtpArgs& a, int pass, int rows, hipStream_t st);
hipError_t launch_rms_rows(const float* in, float* out, int rows, int H, hipStream_t st);
hipError_t launch_mtp_out(const MtpArgs& a, int pass, int rows, int trace_row0, hipStream_t st);

// Gated DeltaNet: one wave per half head (dk = dv = 128).
struct GdnArgs {
  float* S;              // [nh][128][128]
  float* ring;           // [2][nh][T_max-1][258]
  int32_t* n_acc;        // device [2]: accept length of the previous step, ring half
  int use_prev;          // replay n_acc[0] rows (else none)
  const float *q, *k, *v, *g, *beta;  // [T][nh][..]
  float* o;              // [T][nh][128]
  int nh, T, T_max;
};
hipError_t launch_gdn_step(const GdnArgs& a, hipStream_t st);
hipError_t launch_gdn_commit(const GdnArgs& a, hipStream_t st);
}  // namespace mk

// Full-attention decode (mk_attn.hip).
#define MK_ATTN_MAX_G 16
namespace mk {
constexpr int kAttnMaxSplit = 256;  // splits per (agent, KV head)
struct AttnPlan {
  int chunk, smax, n_items;
  int nsplit[MK_ATTN_MAX_G], item0[MK_ATTN_MAX_G + 1];
};
struct AttnArgs {
  const float* q;       // [T][Hq][128]
  const float* gate;    // [T][Hq][128] or null
  float* o;             // [T][Hq][128]
  const uint16_t* k;    // [G][Hkv][cap][128]
  const uint16_t* v;    // [G][Hkv][128][cap]
  const int8_t* k8;     // q8_0 cache: K codes [G][Hkv][cap][128]
  const int8_t* v8;     //             V codes [G][Hkv][cap/64][128][64] (tile-major)
  const uint16_t* ks;   //             K scales [G][Hkv][cap][4]
  const uint16_t* vs;   //             V scales [G][Hkv][cap/32][128]
  float* part_o;        // [T][Hq][smax][128] unnormalised block outputs (4 splits each)
  float* part_ml;       // [T][Hq][smax][2] block max (log2 units) and sum
  float qscale;         // log2(e) / sqrt(128)
  int T, Hq, Hkv, gqa, cap, G, chunk, smax, n_items;
  int ctx[MK_ATTN_MAX_G], gs[MK_ATTN_MAX_G + 1], nsplit[MK_ATTN_MAX_G], item0[MK_ATTN_MAX_G + 1];
};
AttnPlan plan_attn(int G, const int32_t* ctx, const int32_t* gs, int Hkv, int cu_count, bool q8);
size_t attn_workspace_bytes(int T, int Hq, const AttnPlan& p);
// nb = number of 16-column blocks, ceil(max group rows * Hq/Hkv / 16), 1..4.
// q8 selects the q8_0 cache pointers (k8, v8, ks, vs) instead of k, v.
hipError_t launch_attn(AttnArgs a, const AttnPlan& p, int nb, bool q8, void* ws, hipStream_t st);
}  // namespace mk
