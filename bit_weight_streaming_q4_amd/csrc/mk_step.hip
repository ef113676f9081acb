// mk_step.hip — one decode step in ONE persistent cooperative launch.
//
// Pages: richland.au single-stream article, "What shipped" (the whole cycle —
// main model over T = 1 + n_draft rows, lm_head and verification — runs in one
// persistent launch whose phases are separated by a software grid barrier;
// the host reads back only the accepted tokens; the Gated DeltaNet state is
// committed through the accepted token); richland.au 4-agent article, "Why it
// matters" (rows of several agents share one weight read per step).
//
// Phases of a step:
//   prep       q8(x) and the per-tile sums of squares of x (RMSNorm input)
//   per layer  P_in    u  = r(x) * (P_in . q8(x))         -> q8(u)
//              P_out   x += P_out . q8(u)                  -> q8(x), sums of squares
//              gate/up h  = SiLU(r g) * (r u)              -> q8(h)
//              down    x += W_down . q8(h)                 -> q8(x), sums of squares
//              (+ one Gated DeltaNet step per agent in GDN layers, beside the pipeline)
//   lm_prep    hid = r(x) * x, split into fp16 hi + lo fragments
//   lm         logits, per-block argmax, last block: argmax, verify, accept
//              lengths into the GDN states for the next step's replay
// r(x)_t = 1/sqrt(mean(x_t^2) + 1e-6) multiplies the whole dot product of row
// t, so the GEMV runs on q8 of the un-normalised row and the factor is applied
// once in the epilogue.  A phase opens once every tile of its input is
// finished (no grid barrier); the step has one grid barrier, before the lm
// phase.
//
// Roles inside a block of 8 waves (one block per CU):
//   compute waves (4)  Each walks a fixed stream of weight units (64 rows x
//                      one superblock = 9216 B) through all phases of the
//                      step, loading each unit and the activation record of
//                      its superblock into a private 2-slot LDS ring with
//                      LDS-DMA; the first units of the next phase load while
//                      the wave waits for that phase to open.  A wave's
//                      partial sums of a (tile, matrix) go to an LDS mailbox;
//                      it never writes global memory, so its vector-memory
//                      counter only ever holds its own loads.
//   contribution (1)   Sums the block's mailboxes per (tile, matrix) in wave
//                      order, stores one partial per block and counts it on
//                      the tile's ticket.
//   owner (1)          For the tiles the block owns (equal shares per phase):
//                      waits for the ticket, sums the partials in block
//                      order, then RMSNorm factor, SiLU, residual, q8 of the
//                      outputs into the next activation record, sums of
//                      squares; counts its finished tiles; also prep,
//                      lm_prep and the final grid barrier.
//   GDN (1)            The block's Gated DeltaNet half-head jobs of every GDN
//                      layer (nothing in the layer pipeline reads them).
//   watcher (1)        Opens the block's phases: block 0's watcher sums the
//                      finished-tile counters of each producer phase and
//                      writes the number of open phases into every block's
//                      line; the others poll their own line.
// Each GEMV phase is a line of units, tile-major; compute wave w of W takes
// the contiguous stretch [S*w/W, S*(w+1)/W) (the host writes each block's
// plan), so a block's stretch is the union of its waves' and results do not
// depend on timing.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <math.h>
#include <mutex>
#include <vector>

#include "mk.h"
#include "mk_device.h"
#include "mk_lm.h"
#include "mk_gdn.h"
#include "mk_attn.h"
#include "mk_internal.h"

namespace mk {

constexpr int kMaxAgents = 16;
constexpr int kMaxLayers = 128;
constexpr int kTicketTiles = 512;  // tickets per phase instance (max n_out / 64)
constexpr int kTicketStride = 16;  // counters 64 B apart
constexpr int kGdnHeadsPerLayer = 32;
constexpr int kBlock = 512;
constexpr int kWavesPerBlock = kBlock / 64;
constexpr int kCompute = 4;        // compute waves per block (one per SIMD): waves 0..3
constexpr int kServiceWave = 4;    // the block's contributions: mailboxes -> partials, tickets
constexpr int kGdnWave = 5;        // the block's Gated DeltaNet jobs
constexpr int kWatchWave = 6;      // opens phases when their inputs are complete
constexpr int kOwnerWave = 7;      // epilogues of the tiles the block owns, prep, lm_prep
constexpr int kRdySlots = 8;       // finished-tile counters per producer phase (block b adds to b % 8)
constexpr int kRdyStride = 32;     // u32 between counters (one 128-B line each)
// Activation record of one GEMV input, per superblock b (256 values of K),
// kActBytes bytes: the int8 rows in the order the matrix-core A operand reads
// them ([sub-block j][octet q][row t][8 B], rows 0..15, rows >= T zero), then
// s[j][t] and s*gsum[j][t] as floats ([8][16] each).
constexpr int kActA = 8 * 4 * 16 * 8;        // 4096
constexpr int kActBytes = kActA + 2 * 8 * 16 * 4;  // 5120
// An LDS slot holds one weight unit and the activations of its superblock.
constexpr int kSlotBytes = kUnitBytes + kActBytes;
constexpr float kRmsEps = 1e-6f;
constexpr unsigned kSpinLimit = 1u << 26;  // bound of every wait (~seconds)
constexpr int kMaxStamps = 4 * kMaxLayers + 8;
// Bits of the device error word.
constexpr int kErrWatchdog = 1;  // a bounded wait ran out
constexpr int kErrTables = 2;    // the workspace holds another stack's weight table and plans
constexpr int kErrAccept = 4;    // an agent state's accept length was outside 0..T_max-1
// Words of the step's output block (zeroed before each launch).
constexpr int kOutNacc = 16;   // accept length per group
constexpr int kOutTok = 32;    // emitted tokens per row
constexpr int kOutTop = 64;    // argmax per row
constexpr int kOutPass = 96;   // lm streams whose rows are handed over
constexpr int kOutWords = 128;

enum { K_X = 0, K_U = 1, K_X2 = 2, K_H = 3 };

constexpr int kMaxTm = 8;   // (tile, matrix) pairs one block contributes to in one phase
constexpr int kMaxOwn = 4;  // tiles one block owns in one phase
// The work of one block in each of the four phase kinds, computed on the
// host (the unit split has no cheap device-side form: it needs 64-bit
// divisions).
struct BlockPlan {
  int wu[4][kCompute][4];     // per compute wave: first unit, end unit, (tile, matrix) and superblock of the first
  int kp[4][4];               // first contributed (tile, matrix), count, first owned tile, count
  uint8_t tmc[4][kMaxTm][4];  // per contributed pair: first and last compute wave of the block, rank among contributors
  uint8_t oc[4][kMaxOwn][2];  // per owned tile: contributing blocks of matrix 0 and matrix 1
};
constexpr int kPlanWords = (int)(sizeof(BlockPlan) / 4);
static_assert(sizeof(BlockPlan) % 16 == 0, "plans are copied in 16-B words");

// Rows of a partial or mailbox, padded to whole 16-B words.
template <int T>
struct TPad {
  static constexpr int value = (T + 3) & ~3;
};

// Partials loaded per batch in an epilogue: 8, or 6 from 13 rows, where 8
// batches of four row groups do not fit the owner wave's registers beside the
// residual rows and row factors it holds for its tiles.
template <int T>
struct PartBatch {
  static constexpr int value = TPad<T>::value > 16 ? 2 : TPad<T>::value > 12 ? 6 : 8;
};

// More than 16 rows (up to kStepTMax): the activation record of a superblock
// is two 16-row records (rows 0..15, then rows 16..31), each unit runs through
// the 16-row matrix-core engine once per half with its weights held in
// registers, and a compute wave keeps one weight region and two activation
// regions in LDS.
constexpr int kStepTMax = 24;
template <int T>
struct Big {
  static constexpr bool value = T > 16;
};
template <int T>
struct RecBytes {  // bytes per superblock of an activation record
  static constexpr int value = Big<T>::value ? 2 * kActBytes : kActBytes;
};
template <int T>
struct SsRows {  // sums-of-squares slots per 64-column tile
  static constexpr int value = Big<T>::value ? 32 : 16;
};

struct LayerW {
  const uint8_t* w[5];  // p_in, p_out, gate, up, down
};

struct StepArgs {
  int L, H, P, F, V, T, G;
  int gs[MK_LM_MAX_G + 1];
  int Wc;       // compute waves in the grid
  int cmax4;    // byte k: largest number of blocks contributing to one (tile, matrix) of phase kind k
  const LayerW* layers;
  const uint16_t* lm;
  uint64_t gdn_mask[2];
  int8_t gdn_idx[kMaxLayers];
  int n_agents, T_max, nh;
  float* S[kMaxAgents];
  float* ring[kMaxAgents];
  int32_t* nacc[kMaxAgents];
  const float *gq, *gk, *gv, *gg, *gb;
  float* go;
  float* x;
  float* trace;
  const int32_t* drafts;
  // workspace
  unsigned* bar;
  int* err;
  unsigned* tickets;
  unsigned* lm_ticket;
  unsigned* rdy;        // [4L + 1][kRdySlots][kRdyStride]: tiles finished per producer phase (prep, then phase q + 1)
  unsigned* open;       // [grid][kRdyStride]: phases opened for block b (written by block 0's watcher)
  size_t part_half;     // floats per partial buffer (phases alternate between two)
  uint8_t* act;         // activation records, [layer][kind] (see kActBytes)
  size_t act_layer;     // bytes per layer
  size_t act_off[4];    // bytes from the layer's first record, per kind
  float* ss;  // [(2L+1)][H/64][SsRows]
  float* part;
  _Float16* frag;     // lm_head input fragments, one set per 16 rows
  size_t frag_half;   // halves between the sets
  float* lm_val;
  int* lm_idx;
  int32_t* out;  // [0] error word, [16..31] n_acc, [32..63] tokens, [64..95] argmax, [96] first lm pass done
  uint64_t* stamps;  // [kMaxStamps]: block 0's clock after each barrier
  const BlockPlan* plans;  // [grid]
  const uint64_t* ws_tag;  // the workspace's record of the stack whose tables it holds
  uint64_t tag;            // this stack's tag
  float lm_pre;            // exact power-of-two prescale of the lm_head input rows
  // full-attention items, run beside the layer pipeline like the GDN jobs
  int n_attn;                          // attention layers (0: none)
  int attn_Hq, attn_Hkv, attn_gqa, attn_cap, attn_chunk;
  int attn_ctx[kMaxAgents];            // cached positions per agent before this step's rows
  int attn_nsplit[kMaxAgents];         // splits per (agent, KV head)
  int attn_item0[kMaxAgents + 1];      // first item of each agent within a layer
  float attn_qscale;                   // log2(e) / sqrt(128)
  const float* attn_q;                 // [n_attn][T][Hq][128]
  const float* attn_gate;              // [n_attn][T][Hq][128] or null
  const uint16_t* attn_k;              // [n_attn][G][Hkv][cap][128] fp16 (null: q8_0 cache)
  const uint16_t* attn_v;              // [n_attn][G][Hkv][128][cap] fp16
  const int8_t* attn_k8;               // q8_0: [n_attn][G][Hkv][cap][128] codes
  const uint16_t* attn_ks;             //       [n_attn][G][Hkv][cap][4] fp16 scales
  const int8_t* attn_v8;               //       [n_attn][G][Hkv][cap/64][128][64] codes
  const uint16_t* attn_vs;             //       [n_attn][G][Hkv][cap/32][128] fp16 scales
  int attn_q8;                         // the cache is q8_0
  float* attn_o;                       // [n_attn][T][Hq][128]
  float* attn_part;                    // per item: [16 columns][128] outputs, then (max, sum) per column
  unsigned* attn_ticket;               // per (layer, agent, KV head): splits finished, 64 B apart
};

__device__ __forceinline__ bool layer_is_gdn(const StepArgs& a, int l) {
  return (a.gdn_mask[l >> 6] >> (l & 63)) & 1ull;
}

// Keeps loads through p from being issued before this point (the scalar-cache
// reads of a phase's activations must follow the barrier release).
template <typename P>
__device__ __forceinline__ P* fresh(P* p) {
  asm volatile("" : "+s"(p)::"memory");
  return p;
}

// Cross-workgroup data of a step (partials, residual, sums of squares,
// activations) is stored and loaded with device-scope (sc1) accesses;
// ordering comes from waiting for the stores before the ticket or counter
// atomic (ticket_add).  Activations are read through the scalar cache: every
// activation buffer is written once per launch and only read after its
// producer phase, so no stale line can be cached.
//
// 16-B device-scope (sc1) accesses through a buffer resource on a
// wave-uniform base; off is the lane's byte offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
constexpr int kSc1 = 16;  // cache-policy bits of a device-scope access
__device__ __forceinline__ f32x4 ld16(const void* base, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), off, 0, kSc1);
}
__device__ __forceinline__ void st16(void* base, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base), off, 0, kSc1);
}

// Device-coherent reads through the scalar unit (glc): they bypass the
// scalar cache and, unlike vector loads, do not queue behind the weight
// loads the compute waves keep in flight on the same CU.  The address is
// wave-uniform.
__device__ __forceinline__ uint64_t sgpr_addr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ unsigned sld1(const unsigned* p) {
  unsigned v;
  asm volatile("s_load_dword %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(sgpr_addr(p)) : "memory");
  return v;
}
// Sum of the 8 words p[0], p[S], ..., p[7 S] (S = kRdyStride words), all
// loads in flight together.
__device__ __forceinline__ unsigned sld_sum8(const unsigned* p) {
  unsigned v0, v1, v2, v3, v4, v5, v6, v7;
  asm volatile(
      "s_load_dword %0, %8, 0x0 glc\n\t"
      "s_load_dword %1, %8, 0x80 glc\n\t"
      "s_load_dword %2, %8, 0x100 glc\n\t"
      "s_load_dword %3, %8, 0x180 glc\n\t"
      "s_load_dword %4, %8, 0x200 glc\n\t"
      "s_load_dword %5, %8, 0x280 glc\n\t"
      "s_load_dword %6, %8, 0x300 glc\n\t"
      "s_load_dword %7, %8, 0x380 glc\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(v0), "=&s"(v1), "=&s"(v2), "=&s"(v3), "=&s"(v4), "=&s"(v5), "=&s"(v6), "=&s"(v7)
      : "s"(sgpr_addr(p))
      : "memory");
  return v0 + v1 + v2 + v3 + v4 + v5 + v6 + v7;
}
__device__ __forceinline__ u32x8 sld8(const unsigned* p) {
  u32x8 v;
  asm volatile("s_load_dwordx8 %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(sgpr_addr(p)) : "memory");
  return v;
}

// LDS words shared by the waves of a block.  The LDS executes each wave's
// accesses in order, so only the compiler must keep program order (the empty
// asm statements); no wait on the vector-memory counter is involved, which
// keeps a compute wave's weight loads in flight while it polls.
typedef __attribute__((address_space(3))) int lds_int;
__device__ __forceinline__ int lds_ld(const int* p) {
  const int v = __hip_atomic_load((lds_int*)const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  asm volatile("" ::: "memory");
  return v;
}
__device__ __forceinline__ void lds_st(int* p, int v) {
  asm volatile("" ::: "memory");
  __hip_atomic_store((lds_int*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ------------------------------------------------------------ block state
// ring[c][k]: slot k of compute wave c (a 9216-B weight unit and the 5120-B
// activation block of its superblock), filled by the wave's own LDS-DMA loads.  mb[c][k]: mailbox k of compute wave c, the
// partial sums [64][t] of one (tile, matrix) with its tag ((phase + 1) << 16 |
// tile-matrix), 0 when free.  done[c] = phases finished by compute wave c;
// rel = grid barriers completed.  wt: the per-layer weight pointers (read by
// the compute waves at every phase change).  rel = phases opened by the watcher wave
// (phase q is open once every tile of its input is finished).  After the last GEMV phase the ring area
// holds the lm phase's cross-wave reduction.
constexpr int kSlots = 2;
constexpr int kMbRow = 68;  // mailbox row stride in floats: 64 rows + 4 (spreads the flush writes over the banks)
template <int T>
struct MbCount {
  static constexpr int value = Big<T>::value ? 1 : 2;
};
// Per compute wave: two slots of [weights | activations], or above 16 rows
// one weight region and two activation regions of two 16-row halves.
constexpr int kStageBytes = 1024 + 256;  // one tile's part of a 16-row record
template <int T>
struct RingBytes {
  static constexpr int value = Big<T>::value ? kUnitBytes + 2 * RecBytes<T>::value : kSlots * kSlotBytes;
};
template <int T>
struct BlockState {
  static constexpr int NMB = MbCount<T>::value;
  uint8_t ring[kCompute][RingBytes<T>::value] __attribute__((aligned(16)));
  const uint8_t* wt[kMaxLayers][5];  // the weight table, copied at the start
  float mb[kCompute][NMB][TPad<T>::value][kMbRow] __attribute__((aligned(16)));  // [t][row of the tile]
  uint8_t stage[(Big<T>::value ? 2 : 1) * kStageBytes] __attribute__((aligned(16)));  // staged record parts
  BlockPlan plan __attribute__((aligned(16)));
  int tag[kCompute][NMB];
  int done[kCompute];
  int rel;
  int abort;
  int gdn_done;  // the block's Gated DeltaNet jobs have finished
};

// Waits until *p >= v.  A wait that exceeds the bound (or sees another wave
// give up) records the failure and returns false; every later wait then
// falls through and the launch ends without the lm phase.
template <int T>
__device__ __forceinline__ bool wait_ge(const StepArgs& a, BlockState<T>& s, const int* p, int v) {
  unsigned spins = 0;
  while (lds_ld(p) < v) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpinLimit || lds_ld(&s.abort)) {
      lds_st(&s.abort, 1);
      if ((threadIdx.x & 63) == 0) atomicOr(a.err, kErrWatchdog);
      return false;
    }
  }
  return true;
}

// ------------------------------------------------------------ phase lines
struct Line {
  int S;    // units in the phase
  int nsb;  // superblocks per row (units per (tile, matrix))
  int nm;   // matrices sharing the input (gate/up: 2)
  int K, N;
  int W;    // compute waves that share the line: min(all compute waves, S), so none is idle inside it
};

// Opaque copy of a wave-uniform value: a choice among such copies stays a
// choice among values.  (A choice among fields of the argument block would
// become a variable offset into it, which makes the compiler keep a private
// copy of the whole block and read every field through vector memory.)
__device__ __forceinline__ size_t opaque(size_t v) {
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  asm volatile("" : "+s"(lo), "+s"(hi));
  return ((size_t)hi << 32) | lo;
}

__device__ __forceinline__ int opaque_i(int v) {
  v = __builtin_amdgcn_readfirstlane(v);
  asm volatile("" : "+s"(v));
  return v;
}

__device__ __forceinline__ Line line_of(const StepArgs& a, int ph) {
  // opaque copies: the choice below is among values (see opaque())
  const int H = opaque_i(a.H), P = opaque_i(a.P), F = opaque_i(a.F);
  Line ln;
  ln.K = ph == 1 ? P : ph == 3 ? F : H;
  ln.N = ph == 0 ? P : ph == 2 ? F : H;
  ln.nm = ph == 2 ? 2 : 1;
  ln.nsb = ln.K / 256;
  ln.S = (ln.N / 64) * ln.nm * ln.nsb;
  const int Wc = opaque_i(a.Wc);
  ln.W = Wc < ln.S ? Wc : ln.S;
  return ln;
}


// activation record of (layer, kind)
__device__ __forceinline__ uint8_t* act_rec(const StepArgs& a, int layer, int kind) {
  const size_t o0 = opaque(a.act_off[0]), o1 = opaque(a.act_off[1]), o2 = opaque(a.act_off[2]),
               o3 = opaque(a.act_off[3]);
  return a.act + (size_t)layer * a.act_layer + (kind == 0 ? o0 : kind == 1 ? o1 : kind == 2 ? o2 : o3);
}

__device__ __forceinline__ uint8_t* phase_input(const StepArgs& a, int l, int ph) {
  return act_rec(a, l, ph == 0 ? K_X : ph == 1 ? K_U : ph == 2 ? K_X2 : K_H);
}

// Row-group form of a 64-column tile's rows, used by the epilogues: lane
// 16 tr + cq holds rows tr, tr + 4, ... (TP / 4 of them) at columns 4 cq ..
// 4 cq + 3.  A 32-column quantization group is then 8 lanes of one row.
template <int T>
struct RG {
  static constexpr int TP = TPad<T>::value;
  static constexpr int G = TP / 4;  // rows per lane
};

// max / sum over an aligned group of 8 lanes (lane ^ 1, lane ^ 2, half-row
// mirror), and sums over a 16-lane row (plus the row mirror)
__device__ __forceinline__ float max8(float v) {
  v = __builtin_fmaxf(v, dpp_f<0xB1>(v));
  v = __builtin_fmaxf(v, dpp_f<0x4E>(v));
  return __builtin_fmaxf(v, dpp_f<0x141>(v));
}
__device__ __forceinline__ int sum8_i(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  return v + dpp_i<0x141>(v);
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}

// Quantizes the tile's rows (row-group form; rows >= T hold zeros) and
// writes the tile's part of the record: its two sub-blocks' 1024 code bytes
// ([j][q][t][8 B]) and their 2 x 16 scales and scaled code sums.  Both are
// staged in LDS (rows >= TP stay zero there from the start of the launch) so
// that each goes out as one 16-B store per lane.  Group g of row t: lanes
// 16 tr + 8 g .. + 7; each lane's 4 codes are one dword of the record:
// sub-block j = g, octet q = (cq % 8) / 2, bytes 4 (cq % 2) .. + 3.
template <int G>
__device__ __forceinline__ void store_q8_part(uint8_t* blk, int tau, int lane, const f32x4* val, uint8_t* stage) {
  const int tr = lane >> 4, cq = lane & 15;
  const int jj = cq >> 3, q = (cq & 7) >> 1;
  uint8_t* cb = stage + (jj * 4 + q) * 128 + (cq & 1) * 4;
  float* sst = (float*)(stage + 1024);  // [s: 2 x 16][s * gsum: 2 x 16]
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const int t = tr + 4 * k;
    const f32x4 x = val[k];
    float amax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(x[0]), __builtin_fabsf(x[1])),
                                 __builtin_fmaxf(__builtin_fabsf(x[2]), __builtin_fabsf(x[3])));
    amax = max8(amax);
    float sc = amax / 127.0f;
    int c[4] = {0, 0, 0, 0};
    if (sc > 0.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = __builtin_rintf(x[i] / sc);
        c[i] = r == r ? (int)__builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f) : 0;
      }
    } else {
      sc = 0.0f;  // all zero, an underflowing scale, or NaN only: zero codes
    }
    const int gsum = sum8_i(c[0] + c[1] + c[2] + c[3]);
    *(uint32_t*)(cb + t * 8) =
        (uint32_t)(c[0] & 255) | ((uint32_t)(c[1] & 255) << 8) | ((uint32_t)(c[2] & 255) << 16) | ((uint32_t)c[3] << 24);
    if ((cq & 7) == 0) {
      sst[jj * 16 + t] = sc;
      sst[32 + jj * 16 + t] = sc * (float)gsum;
    }
  }
  st16(blk, (tau & 3) * 1024 + lane * 16, *(const f32x4*)(stage + lane * 16));
  if (lane < 16) {
    const int j0 = (tau & 3) * 2;
    const int fo = lane < 8 ? j0 * 16 + lane * 4 : 128 + j0 * 16 + (lane - 8) * 4;
    st16(blk + kActA, fo * 4, *(const f32x4*)(stage + 1024 + lane * 16));
  }
}

// The tile's part of the activation record rec (superblock tau / 4): rows
// 0..15 in the first 16-row record, rows 16..31 (more than 16 rows) in the
// second, each staged in a stage area of its own (its rows above the ones
// written stay zero).
template <int T>
__device__ __forceinline__ void store_q8(uint8_t* rec, int tau, int lane, const f32x4 (&val)[RG<T>::G],
                                         uint8_t* stage) {
  uint8_t* blk = rec + (size_t)(tau >> 2) * RecBytes<T>::value;
  if constexpr (Big<T>::value) {
    store_q8_part<4>(blk, tau, lane, val, stage);
    store_q8_part<RG<T>::G - 4>(blk + kActBytes, tau, lane, val + 4, stage + kStageBytes);
  } else {
    store_q8_part<RG<T>::G>(blk, tau, lane, val, stage);
  }
}

// Sums of squares of the tile's rows (row-group form) into its slots
// (slot t < TP; rows >= T are zero).
template <int T>
__device__ __forceinline__ void store_ss(float* ss16, int lane, const f32x4 (&x)[RG<T>::G]) {
  const int tr = lane >> 4, cq = lane & 15;
#pragma unroll
  for (int k = 0; k < RG<T>::G; ++k) {
    float p = x[k][0] * x[k][0];
    p = __builtin_fmaf(x[k][1], x[k][1], p);
    p = __builtin_fmaf(x[k][2], x[k][2], p);
    p = __builtin_fmaf(x[k][3], x[k][3], p);
    p = sum16(p);
    if (cq == 0) st_coh(ss16 + tr + 4 * k, p);
  }
}

// The tile's rows of x (row-group form), rows >= T zero.
template <int T>
__device__ __forceinline__ void load_rows(const float* x, int H, int tau, int lane, f32x4 (&v)[RG<T>::G]) {
  const int tr = lane >> 4, cq = lane & 15;
#pragma unroll
  for (int k = 0; k < RG<T>::G; ++k) {
    const int t = tr + 4 * k;
    v[k] = t < T ? ld16(x, ((t * H) + tau * 64 + cq * 4) * 4) : (f32x4){0.f, 0.f, 0.f, 0.f};
  }
}

__device__ __forceinline__ int wave_sum_i(int v) { return sum64_i(v); }

// Sum over the 64 lanes (a fixed order; every lane gets the same value).
__device__ __forceinline__ float wave_sum(float v) { return sum64(v); }

// r[t] = 1/sqrt(mean(x_t^2) + eps) from the per-tile sums of squares of
// record ss_idx ([tile][SsRows]): lane i adds tiles i, i+64, ... in order (the
// loads of two such chunks are issued together), then the lanes are summed;
// the same order for every caller.
template <int T>
__device__ __forceinline__ void rnorm_rows(const StepArgs& a, int ss_idx, int lane, float (&r)[T]) {
  constexpr int TP = TPad<T>::value;
  const int ntH = a.H / 64;
  const float* ss = a.ss + (size_t)ss_idx * ntH * SsRows<T>::value;
  f32x4 acc[TP / 4];
#pragma unroll
  for (int i = 0; i < TP / 4; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 * 64 < ntH; k0 += 2) {
    f32x4 v[2][TP / 4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int tile = (k0 + k) * 64 + lane;
      const int tl = tile < ntH ? tile : 0;  // in-range address; the value is not added
#pragma unroll
      for (int i = 0; i < TP / 4; ++i) v[k][i] = ld16(ss, tl * SsRows<T>::value * 4 + i * 16);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if ((k0 + k) * 64 + lane < ntH)
#pragma unroll
        for (int i = 0; i < TP / 4; ++i) acc[i] += v[k][i];
  }
#pragma unroll
  for (int t = 0; t < T; ++t) r[t] = 1.0f / __builtin_sqrtf(wave_sum(acc[t / 4][t % 4]) / (float)a.H + kRmsEps);
}

// ------------------------------------------------------------ compute waves
// Position in the wave's unit stream: phase q (layer q / 4, kind q % 4), the
// units [u, u1) of its stretch still to load, the (tile, matrix) tm and
// superblock b of unit u, and the phase's weight matrices.  q == 4L: ended.
struct Cursor {
  int q, u, u1, tm, b, nsb, nm;
  const uint8_t* W0;
  const uint8_t* W1;
};

// wu: the block plan's unit ranges, [kind][compute wave][4]
typedef const int (*WaveUnits)[kCompute][4];
__device__ __forceinline__ void cursor_settle(const StepArgs& a, const uint8_t* const (*wt)[5], WaveUnits wu, Cursor& c,
                                              int cw) {
  while (c.q < 4 * a.L) {
    const int ph = c.q & 3, l = c.q >> 2;
    const int* p = wu[ph][cw];
    c.u = uniform(p[0]);
    c.u1 = uniform(p[1]);
    if (c.u < c.u1) {
      const Line ln = line_of(a, ph);
      c.nsb = ln.nsb;
      c.nm = ln.nm;
      c.tm = uniform(p[2]);
      c.b = uniform(p[3]);
      const int m0 = ph == 0 ? 0 : ph == 1 ? 1 : ph == 2 ? 2 : 4;
      c.W0 = uniform(wt[l][m0]);
      c.W1 = uniform(wt[l][ph == 2 ? 3 : m0]);
      return;
    }
    ++c.q;
  }
}

// LDS address (for M0) of slot k of compute wave c.
template <int T>
__device__ __forceinline__ uint32_t slot_lds(BlockState<T>& s, int c, int k) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&s.ring[c][k * kSlotBytes];
}

// n LDS-DMA loads of 1 KB (16 B per lane) from global g (this lane's first
// byte) into LDS at byte address lds.  Written in assembly so that the
// compiler neither moves them nor waits for them: the wave waits with
// wait_ops() (its vector-memory operations complete in issue order), and a
// compute wave issues no other vector-memory operation while loads are in
// flight.
// COH: device-scope (sc1) loads, for data other CUs wrote during the launch.
#define MK_DMA1(C) "global_load_lds_dwordx4 %[a], off" C "\n\t"
#define MK_DMA_NEXT "v_lshl_add_u64 %[a], %[a], 0, %[k]\n\ts_add_u32 m0, m0, 0x400\n\t"
#define MK_DMA5(C) MK_DMA1(C) MK_DMA_NEXT MK_DMA1(C) MK_DMA_NEXT MK_DMA1(C) MK_DMA_NEXT MK_DMA1(C) MK_DMA_NEXT MK_DMA1(C)
#define MK_DMA9(C) MK_DMA5(C) MK_DMA_NEXT MK_DMA1(C) MK_DMA_NEXT MK_DMA1(C) MK_DMA_NEXT MK_DMA1(C) MK_DMA_NEXT MK_DMA1(C)
template <int N, bool COH>
__device__ __forceinline__ void dma(uint32_t lds, const uint8_t* g) {
  static_assert((N == 9 && !COH) || N == 5 || (N == 10 && COH), "instantiated shapes only");
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds);
  uint64_t addr = (uint64_t)(uintptr_t)g;
  const uint64_t step = 1024;
  // One statement for all N loads: the address and M0 advance inside it, so
  // no compiler-placed instruction (or wait) falls between the loads.
  if constexpr (N == 9)
    asm volatile("s_mov_b32 m0, %[m]\n\t" MK_DMA9("")
                 : [a] "+v"(addr)
                 : [m] "s"(l0), [k] "s"(step)
                 : "memory", "m0", "scc");
  else if constexpr (N == 5 && !COH)
    asm volatile("s_mov_b32 m0, %[m]\n\t" MK_DMA5("")
                 : [a] "+v"(addr)
                 : [m] "s"(l0), [k] "s"(step)
                 : "memory", "m0", "scc");
  else if constexpr (N == 5)
    asm volatile("s_mov_b32 m0, %[m]\n\t" MK_DMA5(" sc1")
                 : [a] "+v"(addr)
                 : [m] "s"(l0), [k] "s"(step)
                 : "memory", "m0", "scc");
  else
    asm volatile("s_mov_b32 m0, %[m]\n\t" MK_DMA5(" sc1") MK_DMA_NEXT MK_DMA5(" sc1")
                 : [a] "+v"(addr)
                 : [m] "s"(l0), [k] "s"(step)
                 : "memory", "m0", "scc");
}
#undef MK_DMA9
#undef MK_DMA5
#undef MK_DMA_NEXT
#undef MK_DMA1

// Waits until at most n of this wave's vector-memory operations are in flight.
__device__ __forceinline__ void wait_ops(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
  }
}

// One slot of a compute wave: which unit it holds and the vector-memory
// operations its loads still count (weights 9, activations 5).
struct Slot {
  int q, tm, b;
  int wops;    // weight DMA operations issued for this slot's unit
  int aops;    // activation DMA operations issued after them (0 if not yet)
  bool act;    // activations loaded (or in flight)
};

// Starts the weight loads of the cursor's unit into slot lds, records the
// unit and moves the cursor on.
__device__ __forceinline__ void issue_w(const StepArgs& a, const uint8_t* const (*wt)[5], WaveUnits wu, Cursor& c,
                                        int w, int lane, uint32_t lds, Slot& sl) {
  sl.q = c.q;
  sl.tm = c.tm;
  sl.b = c.b;
  sl.wops = 0;
  sl.aops = 0;
  sl.act = false;
  if (c.q >= 4 * a.L) return;
  const int tau = c.nm == 2 ? c.tm >> 1 : c.tm;
  const uint8_t* W = (c.nm == 2 && (c.tm & 1)) ? c.W1 : c.W0;
  dma<9, false>(lds, W + ((size_t)tau * c.nsb + c.b) * kUnitBytes + lane * 16);
  sl.wops = 9;
  if (++c.b == c.nsb) {
    c.b = 0;
    ++c.tm;
  }
  if (++c.u >= c.u1) {
    ++c.q;
    cursor_settle(a, wt, wu, c, w);
  }
}

// Starts the activation loads of slot sl's unit once its phase is open (it
// is the consumer's current phase `open`).  The slot's activation region
// must no longer be read: with WAIT, every LDS read of the wave is waited
// for first; without, the caller has used every value it read.
template <bool WAIT>
__device__ __forceinline__ void issue_a(const StepArgs& a, int lane, uint32_t lds, int open, Slot& sl) {
  if (!sl.wops || sl.act || sl.q != open) return;
  if (WAIT) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  dma<5, true>(lds + kUnitBytes, phase_input(a, sl.q >> 2, sl.q & 3) + (size_t)sl.b * kActBytes + lane * 16);
  sl.aops = 5;
  sl.act = true;
}

// Starts the weight loads of the cursor's unit into slot lds and, if phase
// `open` is the unit's (its activations are ready), its activation loads;
// records the unit and moves the cursor on (the dot4 engine's refill).
__device__ __forceinline__ void issue_wa(const StepArgs& a, const uint8_t* const (*wt)[5], WaveUnits wu, Cursor& c, int w,
                                      int lane, uint32_t lds, int open, Slot& sl) {
  sl.q = c.q;
  sl.tm = c.tm;
  sl.b = c.b;
  sl.wops = 0;
  sl.aops = 0;
  sl.act = false;
  if (c.q >= 4 * a.L) return;
  const int tau = c.nm == 2 ? c.tm >> 1 : c.tm;
  const uint8_t* W = (c.nm == 2 && (c.tm & 1)) ? c.W1 : c.W0;
  dma<9, false>(lds, W + ((size_t)tau * c.nsb + c.b) * kUnitBytes + lane * 16);
  sl.wops = 9;
  if (c.q == open) {
    dma<5, true>(lds + kUnitBytes, phase_input(a, c.q >> 2, c.q & 3) + (size_t)c.b * kActBytes + lane * 16);
    sl.aops = 5;
    sl.act = true;
  }
  if (++c.b == c.nsb) {
    c.b = 0;
    ++c.tm;
  }
  if (++c.u >= c.u1) {
    ++c.q;
    cursor_settle(a, wt, wu, c, w);
  }
}

typedef __attribute__((address_space(3))) const uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;
typedef __attribute__((address_space(3))) const uint64_t lds_u64;
typedef __attribute__((address_space(3))) const float lds_f32;
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;

__device__ __forceinline__ lds_u8* as_lds(const uint8_t* p) { return (lds_u8*)p; }

// dot4 engine on a slot (lane = output row): the unit's codes and header
// from LDS, the activations as wave-uniform LDS reads (every lane the same
// address).  The weight reads stay next to their use: issuing them apart
// from the arithmetic measured slower.
template <int T>
__device__ __forceinline__ void slot_dot4(lds_u8* sl, int lane, float (&acc)[T]) {
  const lds_u32x4* w = (const lds_u32x4*)(sl + lane * 16);
  Unit x;
  x.h = w[0];
#pragma unroll
  for (int j = 0; j < 8; ++j) x.c[j] = w[64 * (j + 1)];
  Hdr hd;
  decode_hdr(x.h, hd);
  lds_u8* act = sl + kUnitBytes;
  lds_f32* sc = (lds_f32*)(act + kActA);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      u32x8 av;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint64_t v = *(lds_u64*)(act + ((j * 4 + q) * 16 + t) * 8);
        av[2 * q] = (uint32_t)v;
        av[2 * q + 1] = (uint32_t)(v >> 32);
      }
      const int p = dot_sub(x.c[j], av);
      acc[t] = __builtin_fmaf((float)p * hd.dsc[j], sc[j * 16 + t], acc[t]);
      acc[t] = __builtin_fmaf(-hd.dm[j], sc[128 + j * 16 + t], acc[t]);
    }
  }
}

// Matrix-core engine on a slot.  Lane l = 16 q + n.  For row group nb (rows
// 16 nb .. 16 nb + 15) and sub-block j, v_mfma_i32_16x16x32_i8 takes the
// activations as A (row t = n, octet q: 8 bytes) and the codes as B (row
// 16 nb + n, octet q: one dword, nibbles widened to bytes) and gives the
// exact sub-block sums P[t = 4q + i][row 16 nb + n].  The combine adds
// s[t][j] * d * sc_j * P, and the min term - dmin * m_j * (s*gsum)[t][j] is a
// v_mfma_f32_16x16x4_f32 over j into the same accumulator.
// LDS operands of sub-block j of the unit in slot sl: the activation A
// fragment, the codes of rows 16 nb + n (dword q) and the scales s of rows
// t = 4q .. 4q + 3.
struct SubOps {
  uint64_t aop;
  f32x4 st;
};

__device__ __forceinline__ void read_sub(lds_u8* act, lds_f32* sc, int j, int q, int n, SubOps& o) {
  o.aop = *(lds_u64*)(act + ((j * 4 + q) * 16 + n) * 8);
  o.st = *(const lds_f32x4*)(sc + j * 16 + 4 * q);
}

// A unit's weights in the matrix-core operand layout: the headers of rows
// 16 nb + n and, per sub-block j, dword q of the codes of those rows.
struct WregM {
  u32x4 h[4];
  uint32_t cw[8][4];
};

__device__ __forceinline__ void read_w_mfma(lds_u8* sl, int lane, WregM& x) {
  const int q = lane >> 4, n = lane & 15;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) x.h[nb] = *(const lds_u32x4*)(sl + (16 * nb + n) * 16);
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      x.cw[j][nb] = *(const lds_u32*)(sl + kHdrBytes + j * kSubBytes + (16 * nb + n) * 16 + q * 4);
}

// Integer products of one sub-block for the 4 row groups: p[nb] = C[t = 4q + i][n].
__device__ __forceinline__ void mfma_sub(const SubOps& o, const uint32_t (&cw)[4], i32x4 (&p)[4]) {
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const uint64_t bop = (uint64_t)(cw[nb] & 0x0F0F0F0Fu) | ((uint64_t)((cw[nb] >> 4) & 0x0F0F0F0Fu) << 32);
    const i32x4 z = {0, 0, 0, 0};
    p[nb] = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)o.aop, (long)bop, z, 0, 0, 0);
  }
}

// Byte k of a dword whose bytes are already below 64, as a float (one
// byte-select conversion).
__device__ __forceinline__ float byte_f32(uint32_t w, int k) { return (float)((w >> (8 * k)) & 0xffu); }

// acc[nb][i] += P * (d * sc_j) * s[t = 4q + i][j] for the products of sub-block j.
__device__ __forceinline__ void scale_sub(int j, const float (&d)[4], const uint32_t (&sc03)[4],
                                          const uint32_t (&sc47)[4], const f32x4 st, const i32x4 (&p)[4],
                                          f32x4 (&acc)[4]) {
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const float f = d[nb] * byte_f32(j < 4 ? sc03[nb] : sc47[nb], j & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nb][i] = __builtin_fmaf((float)p[nb][i], f * st[i], acc[nb][i]);
  }
}

// Matrix-core engine on a unit whose weights are in registers (x), against
// the 16-row activation record at act.
__device__ __forceinline__ void act_mfma(const WregM& x, lds_u8* act, int lane, f32x4 (&acc)[4]) {
  const int q = lane >> 4, n = lane & 15;
  lds_f32* sc = (lds_f32*)(act + kActA);
  const u32x4 (&h)[4] = x.h;
  // activation operands of the first two sub-blocks
  SubOps o0, o1;
  read_sub(act, sc, 0, q, n, o0);
  read_sub(act, sc, 1, q, n, o1);
  float d[4], dmin[4];
  uint32_t sc03[4], sc47[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    d[nb] = f16_bits_to_f32(h[nb].x & 0xffffu);
    dmin[nb] = f16_bits_to_f32(h[nb].x >> 16);
    // masked out of the compiler's sight, so that each scale below is one
    // byte-select conversion rather than a field extract and a conversion
    asm("v_and_b32 %0, %1, %2" : "=v"(sc03[nb]) : "v"(h[nb].y), "v"(0x3F3F3F3Fu));
    asm("v_and_b32 %0, %1, %2" : "=v"(sc47[nb]) : "v"(h[nb].z), "v"(0x3F3F3F3Fu));
  }
  // min term: B[k][n] = -dmin * m_k for k = q (first MFMA) and q + 4 (second)
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const uint32_t m03 = (h[nb].w & 0x0F0F0F0Fu) | ((h[nb].y >> 2) & 0x30303030u);
    const uint32_t m47 = ((h[nb].w >> 4) & 0x0F0F0F0Fu) | ((h[nb].z >> 2) & 0x30303030u);
    const float bm0 = -dmin[nb] * (float)((m03 >> (8 * q)) & 0xffu);
    const float bm1 = -dmin[nb] * (float)((m47 >> (8 * q)) & 0xffu);
    const float am0 = sc[128 + q * 16 + n], am1 = sc[128 + (q + 4) * 16 + n];
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(am0, bm0, acc[nb], 0, 0, 0);
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(am1, bm1, acc[nb], 0, 0, 0);
  }
  // Three stages in flight: the LDS operands of sub-block j + 2 are read and
  // the products of sub-block j + 1 issued before sub-block j is scaled (the
  // loop is unrolled, so every sub-block's values have registers of their own).
  SubOps o[8];
  i32x4 p[8][4];
  o[0] = o0;
  o[1] = o1;
  mfma_sub(o[0], x.cw[0], p[0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j + 2 < 8) read_sub(act, sc, j + 2, q, n, o[j + 2]);
    if (j + 1 < 8) mfma_sub(o[j + 1], x.cw[j + 1], p[j + 1]);
    scale_sub(j, d, sc03, sc47, o[j].st, p[j], acc);
  }
}

// The same on a slot: its activation record follows the unit's weights.
__device__ __forceinline__ void slot_mfma(const WregM& x, lds_u8* sl, int lane, f32x4 (&acc)[4]) {
  act_mfma(x, sl + kUnitBytes, lane, acc);
}

// Matrix-core engine for at most 8 (padded) rows: two sub-blocks per
// v_mfma_i32_16x16x64_i8, in block-diagonal form.  Lane l = 16 q + n, half
// h = q / 2.  In both operands, lane group q carries K chunks 2 (q % 2) and
// 2 (q % 2) + 1 (8 values each) of sub-block 2 jp + h, so the product's rows
// 0..7 are sub-block 2 jp (activation rows t = 0..7, zero where h = 1) and
// rows 8..15 are sub-block 2 jp + 1 (activation rows t = 0..7 placed at 8..15,
// zero where h = 0).  Every output lane then holds a result: lane (q, n) has
// rows t = 4 (q % 2) + i of weight row n for sub-block 2 jp + h, and the two
// halves are added across lanes l and l + 32 when the partial is handed over.
struct WregP {
  u32x4 h[4];
  uint64_t cw[4][4];  // [pair jp][row group nb]: chunks 2 (q % 2), + 1 of sub-block 2 jp + h
};

__device__ __forceinline__ void read_w_pk(lds_u8* sl, int lane, WregP& x) {
  const int q = lane >> 4, n = lane & 15, hh = q >> 1;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) x.h[nb] = *(const lds_u32x4*)(sl + (16 * nb + n) * 16);
#pragma unroll
  for (int jp = 0; jp < 4; ++jp)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      x.cw[jp][nb] = *(lds_u64*)(sl + kHdrBytes + (2 * jp + hh) * kSubBytes + (16 * nb + n) * 16 + (q & 1) * 8);
}

struct SubOpsP {
  u32x4 aop;  // 16 activation bytes (zero off the diagonal)
  f32x4 st;   // s of rows t = 4 (q % 2) .. + 3 of sub-block 2 jp + h
};

// Off-diagonal lanes read row 15 of the record, which is zero for T <= 8.
__device__ __forceinline__ void read_sub_pk(lds_u8* act, lds_f32* sc, int jp, int q, int n, SubOpsP& o) {
  const int hh = q >> 1;
  const bool diag = (n < 8) == (hh == 0);
  const int tt = diag ? n - 8 * hh : 15;
  const int jj = 2 * jp + hh, c0 = 2 * (q & 1);
  const uint64_t a0 = *(lds_u64*)(act + ((jj * 4 + c0) * 16 + tt) * 8);
  const uint64_t a1 = *(lds_u64*)(act + ((jj * 4 + c0 + 1) * 16 + tt) * 8);
  o.aop = (u32x4){(uint32_t)a0, (uint32_t)(a0 >> 32), (uint32_t)a1, (uint32_t)(a1 >> 32)};
  o.st = *(const lds_f32x4*)(sc + jj * 16 + 4 * (q & 1));
}

__device__ __forceinline__ void mfma_sub_pk(const SubOpsP& o, const uint64_t (&cw)[4], i32x4 (&p)[4]) {
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const uint32_t w0 = (uint32_t)cw[nb], w1 = (uint32_t)(cw[nb] >> 32);
    const u32x4 b = {w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
    const i32x4 z = {0, 0, 0, 0};
    p[nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, o.aop), __builtin_bit_cast(i32x4, b), z,
                                                  0, 0, 0);
  }
}

// acc[nb][i] += P * (d * sc) * s for the products of pair jp; sc03h/sc47h hold
// this lane's sub-block scales shifted so that byte 2 (jp % 2) is sub-block
// 2 jp + h.
__device__ __forceinline__ void scale_sub_pk(int jp, const float (&d)[4], const uint32_t (&sc03h)[4],
                                             const uint32_t (&sc47h)[4], const f32x4 st, const i32x4 (&p)[4],
                                             f32x4 (&acc)[4]) {
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const float f = d[nb] * byte_f32(jp < 2 ? sc03h[nb] : sc47h[nb], 2 * (jp & 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nb][i] = __builtin_fmaf((float)p[nb][i], f * st[i], acc[nb][i]);
  }
}

__device__ __forceinline__ void slot_mfma_pk(const WregP& x, lds_u8* sl, int lane, f32x4 (&acc)[4]) {
  const int q = lane >> 4, n = lane & 15, hh = q >> 1;
  lds_u8* act = sl + kUnitBytes;
  lds_f32* sc = (lds_f32*)(act + kActA);
  const u32x4 (&h)[4] = x.h;
  SubOpsP o[4];
  read_sub_pk(act, sc, 0, q, n, o[0]);
  read_sub_pk(act, sc, 1, q, n, o[1]);
  float d[4], dmin[4];
  uint32_t sc03[4], sc47[4], sc03h[4], sc47h[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    d[nb] = f16_bits_to_f32(h[nb].x & 0xffffu);
    dmin[nb] = f16_bits_to_f32(h[nb].x >> 16);
    asm("v_and_b32 %0, %1, %2" : "=v"(sc03[nb]) : "v"(h[nb].y), "v"(0x3F3F3F3Fu));
    asm("v_and_b32 %0, %1, %2" : "=v"(sc47[nb]) : "v"(h[nb].z), "v"(0x3F3F3F3Fu));
    sc03h[nb] = sc03[nb] >> (8 * hh);
    sc47h[nb] = sc47[nb] >> (8 * hh);
  }
  // min term, as in slot_mfma: its rows t >= 8 have zero activation sums, so
  // it lands in lanes q < 2 only
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const uint32_t m03 = (h[nb].w & 0x0F0F0F0Fu) | ((h[nb].y >> 2) & 0x30303030u);
    const uint32_t m47 = ((h[nb].w >> 4) & 0x0F0F0F0Fu) | ((h[nb].z >> 2) & 0x30303030u);
    const float bm0 = -dmin[nb] * (float)((m03 >> (8 * q)) & 0xffu);
    const float bm1 = -dmin[nb] * (float)((m47 >> (8 * q)) & 0xffu);
    const float am0 = sc[128 + q * 16 + n], am1 = sc[128 + (q + 4) * 16 + n];
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(am0, bm0, acc[nb], 0, 0, 0);
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(am1, bm1, acc[nb], 0, 0, 0);
  }
  i32x4 p[4][4];
  mfma_sub_pk(o[0], x.cw[0], p[0]);
#pragma unroll
  for (int jp = 0; jp < 4; ++jp) {
    if (jp + 2 < 4) read_sub_pk(act, sc, jp + 2, q, n, o[jp + 2]);
    if (jp + 1 < 4) mfma_sub_pk(o[jp + 1], x.cw[jp + 1], p[jp + 1]);
    scale_sub_pk(jp, d, sc03h, sc47h, o[jp].st, p[jp], acc);
  }
}

// Which engine a T-row instance uses: dot4 for one row (its arithmetic is
// short enough to hide under the loads), the packed matrix-core engine up to
// 8 padded rows, the plain one above.
template <int T>
struct UseMfma {
  static constexpr bool value = T > 1;
};
template <int T>
struct PackMfma {
  static constexpr bool value = UseMfma<T>::value && TPad<T>::value <= 8;
};

// What a compute wave accumulates: the open (tile, matrix) of phase q.  The
// dot4 engine keeps row = lane, T rows (acc); the matrix-core engine keeps
// the 4 row groups x 4 rows t of the C layout (macc).
template <int T>
struct Consumer {
  int q;      // current phase (-1 before the first)
  int tm;     // open (tile, matrix), -1 if none
  int nflush;
  int done;   // phases reported finished
  float acc[T];
  f32x4 macc[4];
  f32x4 macc2[4];  // rows 16..31 (more than 16 rows)
};

template <int T>
__device__ __forceinline__ void acc_zero(Consumer<T>& k) {
#pragma unroll
  for (int t = 0; t < T; ++t) k.acc[t] = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) k.macc[nb] = k.macc2[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// Writes the open partial to the wave's mailbox as [t][64 rows of the tile].
template <int T>
__device__ __forceinline__ void flush(BlockState<T>& s, int c, int lane, Consumer<T>& k, bool& ok) {
  const int slot = BlockState<T>::NMB == 2 ? (k.nflush & 1) : 0;
  // a mailbox is free when its tag is 0
  unsigned spins = 0;
  while (ok && lds_ld(&s.tag[c][slot]) != 0) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpinLimit || lds_ld(&s.abort)) {
      lds_st(&s.abort, 1);  // the service wave reports the failure
      ok = false;
    }
  }
  if constexpr (UseMfma<T>::value) {
    if constexpr (PackMfma<T>::value) {
      // the packed engine's lanes l + 32 hold the second sub-block of each pair
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) k.macc[nb][i] += __shfl_xor(k.macc[nb][i], 32, 64);
    }
    // C layout: lane 16 q + n holds rows t = 4q .. 4q + 3 of tile row 16 nb + n
    const int q = lane >> 4, n = lane & 15;
    if (4 * q < TPad<T>::value)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s.mb[c][slot][4 * q + i][16 * nb + n] = k.macc[nb][i];
    if constexpr (Big<T>::value) {
      if (16 + 4 * q < TPad<T>::value)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s.mb[c][slot][16 + 4 * q + i][16 * nb + n] = k.macc2[nb][i];
    }
  } else {
#pragma unroll
    for (int t = 0; t < T; ++t) s.mb[c][slot][t][lane] = k.acc[t];
  }
  if (lane == 0) lds_st(&s.tag[c][slot], ((k.q + 1) << 16) | k.tm);
  ++k.nflush;
  k.tm = -1;
}

// LDS-only wait (a compute wave issues no global atomics: the service wave
// reports failures).
template <int T>
__device__ __forceinline__ bool cw_wait_ge(BlockState<T>& s, const int* p, int v) {
  unsigned spins = 0;
  while (lds_ld(p) < v) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpinLimit || lds_ld(&s.abort)) {
      lds_st(&s.abort, 1);
      return false;
    }
  }
  return true;
}

// Ends phases until phase q is current: flushes the open partial, reports
// each finished phase and waits for the barrier that opens the next one.
template <int T>
__device__ __forceinline__ void advance_to(const StepArgs& a, BlockState<T>& s, int c, int lane, Consumer<T>& k,
                                           int q, bool& ok) {
  while (k.q < q) {
    if (k.q >= 0) {
      if (k.tm >= 0) flush<T>(s, c, lane, k, ok);
      if (k.done < k.q + 1) {
        k.done = k.q + 1;
        if (lane == 0) lds_st(&s.done[c], k.done);
      }
    }
    ++k.q;
    if (k.q < 4 * a.L) ok = ok && cw_wait_ge(s, &s.rel, k.q + 1);
  }
}

// After a unit: if the next unit (nq, ntm) of the stream leaves the open
// (tile, matrix) or the phase, hand over the partial now and report the
// finished phase, so the service wave does not wait for the next unit's
// bookkeeping.
template <int T>
__device__ __forceinline__ void finish_early(BlockState<T>& s, int c, int lane, Consumer<T>& k, int nq, int ntm,
                                             bool& ok) {
  if (k.tm >= 0 && (nq != k.q || ntm != k.tm)) flush<T>(s, c, lane, k, ok);
  if (nq != k.q && k.done < k.q + 1) {
    k.done = k.q + 1;
    if (lane == 0) lds_st(&s.done[c], k.done);
  }
}

// The dot4 engine's stream (T = 1): as below, but each slot is refilled
// after its unit's arithmetic, which measured faster for this short
// arithmetic.  Consumes the unit of slot `cur` (the other slot `oth` holds
// the next one).
// Entering a new phase: wait for its barrier, then start the activation
// loads of both slots' units of that phase, and wait for all loads.
template <int T>
__device__ __forceinline__ void consume_dot4(const StepArgs& a, BlockState<T>& s, int c, int lane, Consumer<T>& k,
                                        Slot& cur, Slot& oth, int kcur, uint32_t lcur, uint32_t loth, bool& ok) {
  if (cur.q != k.q) {
    advance_to<T>(a, s, c, lane, k, cur.q, ok);
    if (!cur.act) {
      dma<5, true>(lcur + kUnitBytes, phase_input(a, cur.q >> 2, cur.q & 3) + (size_t)cur.b * kActBytes + lane * 16);
      cur.act = true;
    }
    if (oth.q == cur.q && oth.wops && !oth.act) {
      dma<5, true>(loth + kUnitBytes, phase_input(a, oth.q >> 2, oth.q & 3) + (size_t)oth.b * kActBytes + lane * 16);
      oth.act = true;
    }
    wait_ops(0);
  } else {
    wait_ops(oth.wops + oth.aops);  // this slot's loads are older than the other slot's
  }
  if (cur.tm != k.tm) {
    if (k.tm >= 0) flush<T>(s, c, lane, k, ok);
    k.tm = cur.tm;
    acc_zero<T>(k);
  }
  lds_u8* sl = as_lds(&s.ring[c][kcur * kSlotBytes]);
  slot_dot4<T>(sl, lane, k.acc);
}

template <int T>
__device__ __forceinline__ void compute_wave_dot4(const StepArgs& a, BlockState<T>& s, int c, int lane) {
  const int w = c;  // the plan indexes compute waves within the block
  const int qend = 4 * a.L;
  const uint32_t l0 = slot_lds(s, c, 0), l1 = slot_lds(s, c, 1);
  const uint8_t* const(*wt)[5] = s.wt;
  WaveUnits wu = s.plan.wu;
  Cursor cur;
  cur.q = 0;
  cursor_settle(a, wt, wu, cur, w);
  Slot s0, s1;
  issue_wa(a, wt, wu, cur, w, lane, l0, -1, s0);
  issue_wa(a, wt, wu, cur, w, lane, l1, -1, s1);
  Consumer<T> k;
  k.q = -1;
  k.tm = -1;
  k.nflush = 0;
  k.done = 0;
  acc_zero<T>(k);
  bool ok = true;
  while (ok) {
    if (s0.q >= qend) break;
    consume_dot4<T>(a, s, c, lane, k, s0, s1, 0, l0, l1, ok);
    finish_early<T>(s, c, lane, k, s1.q, s1.tm, ok);
    // the slot's LDS reads have completed (their values were used) before it is refilled
    issue_wa(a, wt, wu, cur, w, lane, l0, k.q, s0);
    if (s1.q >= qend) break;
    consume_dot4<T>(a, s, c, lane, k, s1, s0, 1, l1, l0, ok);
    finish_early<T>(s, c, lane, k, s0.q, s0.tm, ok);
    issue_wa(a, wt, wu, cur, w, lane, l1, k.q, s1);
  }
  advance_to<T>(a, s, c, lane, k, qend, ok);  // finishes the phases after the last unit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load outlives the stream (also after an abort)
}

// Consumes the unit of slot `cur` (the other slot `oth` holds the next one).
// Entering a new phase: wait for it to open, then start the activation
// loads of both slots' units of that phase, and wait for all loads.  The
// unit's weights are copied into registers and the slot's weight region is
// refilled with the stream's next unit before the matrix-core arithmetic
// starts; the activation region is refilled after it.
template <int T>
__device__ __forceinline__ void consume(const StepArgs& a, BlockState<T>& s, int c, int lane, Consumer<T>& k,
                                        const uint8_t* const (*wt)[5], WaveUnits wu, Cursor& cs, Slot& cur,
                                        Slot& oth, int kcur, uint32_t lcur, uint32_t loth, bool& ok) {
  if (cur.q != k.q) {
    advance_to<T>(a, s, c, lane, k, cur.q, ok);
    if (!cur.act) {
      dma<5, true>(lcur + kUnitBytes, phase_input(a, cur.q >> 2, cur.q & 3) + (size_t)cur.b * kActBytes + lane * 16);
      cur.act = true;
    }
    if (oth.q == cur.q && oth.wops && !oth.act) {
      dma<5, true>(loth + kUnitBytes, phase_input(a, oth.q >> 2, oth.q & 3) + (size_t)oth.b * kActBytes + lane * 16);
      oth.aops = 5;
      oth.act = true;
    }
    wait_ops(0);
  } else {
    wait_ops(oth.wops + oth.aops);  // issued after this slot's loads: the other slot's
  }
  if (cur.tm != k.tm) {
    if (k.tm >= 0) flush<T>(s, c, lane, k, ok);
    k.tm = cur.tm;
    acc_zero<T>(k);
  }
  lds_u8* sl = as_lds(&s.ring[c][kcur * kSlotBytes]);
  if constexpr (PackMfma<T>::value) {
    WregP x;
    read_w_pk(sl, lane, x);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the weight region is read before it is refilled
    issue_w(a, wt, wu, cs, c, lane, lcur, cur);
    slot_mfma_pk(x, sl, lane, k.macc);
  } else {
    WregM x;
    read_w_mfma(sl, lane, x);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the weight region is read before it is refilled
    issue_w(a, wt, wu, cs, c, lane, lcur, cur);
    slot_mfma(x, sl, lane, k.macc);
  }
  finish_early<T>(s, c, lane, k, oth.q, oth.tm, ok);
  issue_a<true>(a, lane, lcur, k.q, cur);
}

template <int T>
__device__ __forceinline__ void compute_wave_mfma(const StepArgs& a, BlockState<T>& s, int c, int lane) {
  const int w = c;  // the plan indexes compute waves within the block
  const int qend = 4 * a.L;
  const uint32_t l0 = slot_lds(s, c, 0), l1 = slot_lds(s, c, 1);
  const uint8_t* const(*wt)[5] = s.wt;
  WaveUnits wu = s.plan.wu;
  Cursor cur;
  cur.q = 0;
  cursor_settle(a, wt, wu, cur, w);
  Slot s0, s1;
  issue_w(a, wt, wu, cur, w, lane, l0, s0);
  issue_w(a, wt, wu, cur, w, lane, l1, s1);
  Consumer<T> k;
  k.q = -1;
  k.tm = -1;
  k.nflush = 0;
  k.done = 0;
  acc_zero<T>(k);
  bool ok = true;
  while (ok) {
    if (s0.q >= qend) break;
    consume<T>(a, s, c, lane, k, wt, wu, cur, s0, s1, 0, l0, l1, ok);
    if (s1.q >= qend) break;
    consume<T>(a, s, c, lane, k, wt, wu, cur, s1, s0, 1, l1, l0, ok);
  }
  advance_to<T>(a, s, c, lane, k, qend, ok);  // finishes the phases after the last unit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load outlives the stream (also after an abort)
}

// More than 16 rows: one weight region and two activation regions per
// compute wave (unit n's activations in region n % 2).  Consuming unit n:
// wait for its loads, issued while unit n - 1 was computed; copy its weights
// into registers; issue the next unit's weights into the weight region and,
// if the next unit's phase is open, its activations into the other region;
// then run the 16-row engine on rows 0..15 and on rows 16..31 of the record.
// Entering a new phase: wait for it to open and start the unit's activation
// loads first.
template <int T>
__device__ __forceinline__ void consume_big(const StepArgs& a, BlockState<T>& s, int c, int lane, Consumer<T>& k,
                                            const uint8_t* const (*wt)[5], WaveUnits wu, Cursor& cs, Slot& cur,
                                            Slot& nxt, uint32_t lw, uint32_t lcur, uint32_t lnxt, lds_u8* wreg,
                                            lds_u8* acur, bool& ok) {
  if (cur.q != k.q) advance_to<T>(a, s, c, lane, k, cur.q, ok);
  if (!cur.act) {
    dma<10, true>(lcur, phase_input(a, cur.q >> 2, cur.q & 3) + (size_t)cur.b * RecBytes<T>::value + lane * 16);
    cur.act = true;
  }
  wait_ops(0);
  if (cur.tm != k.tm) {
    if (k.tm >= 0) flush<T>(s, c, lane, k, ok);
    k.tm = cur.tm;
    acc_zero<T>(k);
  }
  WregM x;
  read_w_mfma(wreg, lane, x);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the weight region is read before it is refilled
  issue_w(a, wt, wu, cs, c, lane, lw, nxt);
  // the other activation region held the previous unit, whose arithmetic is done
  if (nxt.wops && nxt.q == k.q) {
    dma<10, true>(lnxt, phase_input(a, nxt.q >> 2, nxt.q & 3) + (size_t)nxt.b * RecBytes<T>::value + lane * 16);
    nxt.act = true;
  }
  act_mfma(x, acur, lane, k.macc);
  act_mfma(x, acur + kActBytes, lane, k.macc2);
  finish_early<T>(s, c, lane, k, nxt.q, nxt.tm, ok);
}

template <int T>
__device__ __forceinline__ void compute_wave_big(const StepArgs& a, BlockState<T>& s, int c, int lane) {
  const int qend = 4 * a.L;
  uint8_t* base = &s.ring[c][0];
  const uint32_t lw = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)base;
  const uint32_t la0 = lw + kUnitBytes, la1 = la0 + RecBytes<T>::value;
  lds_u8* wreg = as_lds(base);
  lds_u8* a0 = as_lds(base + kUnitBytes);
  lds_u8* a1 = as_lds(base + kUnitBytes + RecBytes<T>::value);
  const uint8_t* const(*wt)[5] = s.wt;
  WaveUnits wu = s.plan.wu;
  Cursor cur;
  cur.q = 0;
  cursor_settle(a, wt, wu, cur, c);
  Slot s0, s1;
  issue_w(a, wt, wu, cur, c, lane, lw, s0);
  s1.q = qend;
  s1.tm = -1;
  s1.b = 0;
  s1.wops = 0;
  s1.aops = 0;
  s1.act = false;
  Consumer<T> k;
  k.q = -1;
  k.tm = -1;
  k.nflush = 0;
  k.done = 0;
  acc_zero<T>(k);
  bool ok = true;
  while (ok) {
    if (s0.q >= qend) break;
    consume_big<T>(a, s, c, lane, k, wt, wu, cur, s0, s1, lw, la0, la1, wreg, a0, ok);
    if (s1.q >= qend) break;
    consume_big<T>(a, s, c, lane, k, wt, wu, cur, s1, s0, lw, la1, la0, wreg, a1, ok);
  }
  advance_to<T>(a, s, c, lane, k, qend, ok);  // finishes the phases after the last unit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load outlives the stream (also after an abort)
}

// A compute wave's stream of units through every phase of the step.
template <int T>
__device__ __forceinline__ void compute_wave(const StepArgs& a, BlockState<T>& s, int c, int lane) {
  if constexpr (Big<T>::value)
    compute_wave_big<T>(a, s, c, lane);
  else if constexpr (UseMfma<T>::value)
    compute_wave_mfma<T>(a, s, c, lane);
  else
    compute_wave_dot4<T>(a, s, c, lane);
}

__device__ __forceinline__ void gdn_job(const StepArgs& a, int layer, long j, int lane) {
  const int agent = (int)(j / (kGdnHeadsPerLayer * 2));
  const int head = (int)((j / 2) % kGdnHeadsPerLayer);
  const int half = (int)(j & 1);
  // per-agent values indexed from the argument block: make them wave-uniform
  const int hh = uniform((int)a.gdn_idx[layer]) * kGdnHeadsPerLayer + head;
  const int32_t* na = uniform(a.nacc[agent]);
  const int par = *as_const<int32_t>(na + 1) & 1;
  const int r0 = uniform(a.gs[agent]);
  const int r1 = uniform(a.gs[agent + 1]);
  float* const Sa = uniform(a.S[agent]);
  float* const Ra = uniform(a.ring[agent]);
  GdnHalf x;
  x.S = Sa + (size_t)hh * kD * kD;
  x.ring_rd = Ra + ((size_t)par * a.nh + hh) * (a.T_max - 1) * kRingRow;
  x.ring_wr = Ra + ((size_t)(par ^ 1) * a.nh + hh) * (a.T_max - 1) * kRingRow;
  x.nrep = checked_acc(const_cast<int32_t*>(na), a.T_max, lane == 0);
  if (x.nrep != *as_const<int32_t>(na) && lane == 0) atomicOr(a.err, kErrAccept);  // nothing replayed
  x.q = a.gq + ((size_t)r0 * a.nh + hh) * kD;
  x.k = a.gk + ((size_t)r0 * a.nh + hh) * kD;
  x.v = a.gv + ((size_t)r0 * a.nh + hh) * kD;
  x.g = a.gg + (size_t)r0 * a.nh + hh;
  x.beta = a.gb + (size_t)r0 * a.nh + hh;
  x.sqk = (size_t)a.nh * kD;
  x.sv = (size_t)a.nh * kD;
  x.sgb = a.nh;
  x.o = a.go + ((size_t)r0 * a.nh + hh) * kD;
  x.so = (size_t)a.nh * kD;
  x.T = r1 - r0;
  x.half = half;
  gdn_half_step(x, lane);
}

// ------------------------------------------------------------ service wave
// Grid barrier k (0-based): the block arrives once its compute waves have
// finished `done` phases and this wave's stores have completed; the wave spins
// on the counter with device-scope loads and then opens the next phase for
// its block (rel = k + 1).  The counter only grows within a launch (zeroed
// before it), so barrier k waits for (k + 1) * gridDim.x arrivals.
template <int T>
__device__ __forceinline__ bool svc_barrier(const StepArgs& a, BlockState<T>& s, int k, int done, int lane, bool ok,
                                            int rel_val) {
  for (int c = 0; c < kCompute && ok; ++c) ok = wait_ge(a, s, &s.done[c], done);
  if (!ok) return false;
  const unsigned target = (unsigned)(k + 1) * gridDim.x;
  int fail = 0;
  if (lane == 0) {
    ticket_add(a.bar);
    unsigned spins = 0;
    while (__hip_atomic_load(a.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      // another block giving up (its watchdog bit) ends this wait too; the
      // other bits report conditions the step runs through
      if (++spins > kSpinLimit ||
          (__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kErrWatchdog)) {
        atomicOr(a.err, kErrWatchdog);
        fail = 1;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (blockIdx.x == 0 && rel_val < kMaxStamps) a.stamps[rel_val] = wall_clock64();
  }
  fail = __shfl(fail, 0, 64);
  if (fail) {
    lds_st(&s.abort, 1);
    return false;
  }
  if (lane == 0) lds_st(&s.rel, rel_val);
  return true;
}

template <int T>
__device__ __forceinline__ void svc_prep(const StepArgs& a, int lane, uint8_t* stage) {
  const int ntH = a.H / 64;
  for (int tau = blockIdx.x; tau < ntH; tau += gridDim.x) {
    f32x4 xv[RG<T>::G];
    load_rows<T>(a.x, a.H, tau, lane, xv);
    store_ss<T>(a.ss + (size_t)tau * SsRows<T>::value, lane, xv);
    store_q8<T>(act_rec(a, 0, K_X), tau, lane, xv, stage);
  }
  const int n = ntH > (int)blockIdx.x ? (ntH - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  if (n) {
    stores_done();
    if (lane == 0) __hip_atomic_fetch_add(a.rdy + (blockIdx.x % kRdySlots) * kRdyStride, (unsigned)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Sum of the block partials of (tile, matrix) pairs tau*nm + m, m < nm (n0
// and n1 contributing blocks), in block order, in row-group form; all loads
// of up to PartBatch partials are issued together.  A partial is
// [TP rows][64 columns].
template <int T>
__device__ __forceinline__ void sum_partials(const StepArgs& a, int q, int nm, int tau, int n0, int n1, int lane,
                                             f32x4 (&v0)[RG<T>::G], f32x4 (&v1)[RG<T>::G]) {
  constexpr int TP = RG<T>::TP, G = RG<T>::G;
  const int ph = q & 3;
  const float* part = a.part + (size_t)(q & 1) * a.part_half;
  const int tm0 = tau * nm;
  const int n = n0 + n1, cm = (a.cmax4 >> (8 * ph)) & 255;
  const int lo = ((lane >> 4) * 64 + (lane & 15) * 4) * 4;  // bytes: row tr, column 4 cq
#pragma unroll
  for (int k = 0; k < G; ++k) v0[k] = v1[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
  constexpr int B = PartBatch<T>::value;
  for (int e0 = 0; e0 < n; e0 += B) {
    f32x4 tmp[B][G];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int e = e0 + i < n ? e0 + i : n - 1;  // in-range address; extra values are not added
      const int m = e < n0 ? 0 : 1, r = e < n0 ? e : e - n0;
      const int off = ((tm0 + m) * cm + r) * TP * 64 * 4 + lo;
#pragma unroll
      for (int k = 0; k < G; ++k) tmp[i][k] = ld16(part, off + k * 4 * 64 * 4);
    }
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (e0 + i >= n) break;
#pragma unroll
      for (int k = 0; k < G; ++k) {
        if (e0 + i < n0)
          v0[k] += tmp[i][k];
        else
          v1[k] += tmp[i][k];
      }
    }
  }
}

// The epilogue of tile tau of phase q, run by the tile's owner once every
// contribution is in: r[t] (RMSNorm factors of the phase input, phases 0
// and 2) and xo[t] (the residual rows of the tile, phases 1 and 3) were
// loaded at the start of the phase.
template <int T>
__device__ __forceinline__ void svc_epilogue(const StepArgs& a, int q, int tau, int n0, int n1, int lane,
                                             const f32x4 (&r)[RG<T>::G], const f32x4 (&xo)[RG<T>::G],
                                             uint8_t* stage) {
  constexpr int G = RG<T>::G;
  const int l = q >> 2, ph = q & 3;
  const int tr = lane >> 4, cq = lane & 15;
  f32x4 v0[G], v1[G];
  sum_partials<T>(a, q, ph == 2 ? 2 : 1, tau, n0, n1, lane, v0, v1);
  // rows >= T of a partial are not results (the dot-product engine leaves them unset)
#pragma unroll
  for (int k = 0; k < G; ++k)
    if (tr + 4 * k >= T) v0[k] = v1[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (ph == 0 || ph == 2) {
    f32x4 y[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (ph == 0) {
          y[k][i] = r[k][i] * v0[k][i];
        } else {
          const float g = r[k][i] * v0[k][i], u = r[k][i] * v1[k][i];
          y[k][i] = g * u / (1.0f + expf(-g));
        }
      }
    }
    store_q8<T>(act_rec(a, l, ph == 0 ? K_U : K_H), tau, lane, y, stage);
  } else {
    f32x4 xn[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      xn[k] = xo[k] + v0[k];
      const int t = tr + 4 * k;
      if (t < T) {
        st16(a.x, (t * a.H + tau * 64 + cq * 4) * 4, xn[k]);
        if (ph == 3 && a.trace) *(f32x4*)(a.trace + ((size_t)l * T + t) * a.H + tau * 64 + cq * 4) = xn[k];
      }
    }
    const int ss_idx = ph == 1 ? 2 * l + 1 : 2 * l + 2;
    store_ss<T>(a.ss + ((size_t)ss_idx * (a.H / 64) + tau) * SsRows<T>::value, lane, xn);
    if (ph == 1)
      store_q8<T>(act_rec(a, l, K_X2), tau, lane, xn, stage);
    else if (l + 1 < a.L)
      store_q8<T>(act_rec(a, l + 1, K_X), tau, lane, xn, stage);
  }
}

// One GEMV phase seen from the service wave of block b.  Tiles are owned by
// blocks in equal shares (tile tau by block tau * G / n_tiles), whatever
// blocks contribute to them.  At the start of the phase the owner loads what
// its epilogues need besides the partials (row factors or residual rows).
// Then: wait for the compute waves' mailboxes of each (tile, matrix) the
// block touches, sum them in wave order, store the block partial, count the
// contributions on the tiles' tickets (one atomic per tile), and, as owner,
// wait for each owned tile's count to complete and run its epilogue.
template <int T>
__device__ __forceinline__ bool svc_contrib(const StepArgs& a, BlockState<T>& s, int q, int lane, bool ok) {
  constexpr int TP = TPad<T>::value;
  const int l = q >> 2, ph = q & 3;
  const int nm = ph == 2 ? 2 : 1;
  const int tm0 = uniform(s.plan.kp[ph][0]), ntm = uniform(s.plan.kp[ph][1]);
  const int own0 = uniform(s.plan.kp[ph][2]), nown = uniform(s.plan.kp[ph][3]);
  if (!wait_ge(a, s, &s.rel, q + 1)) return false;
  if (!ok) return ok;
  unsigned* tk = a.tickets + ((size_t)l * 4 + ph) * kTicketTiles * kTicketStride;
  if (ntm > 0) {
    const int cm = (a.cmax4 >> (8 * ph)) & 255;
    float* part = a.part + (size_t)(q & 1) * a.part_half;
    for (int i = 0; i < ntm; ++i) {
      const int tm = tm0 + i;
      const uint32_t pc = uniform(*(const uint32_t*)&s.plan.tmc[ph][i][0]);
      const int c_lo = pc & 255, c_hi = (pc >> 8) & 255, rank = (pc >> 16) & 255;
      const int want = ((q + 1) << 16) | tm;
      // lane NMB*c + k watches mailbox k of compute wave c
      constexpr int NMB = BlockState<T>::NMB;
      constexpr uint64_t kAll = (1ull << NMB) - 1;
      uint64_t have = 0;
      unsigned spins = 0;
      while (true) {
        const int tg = lane < NMB * kCompute ? lds_ld(&s.tag[lane / NMB][lane % NMB]) : 0;
        have = __ballot(tg == want);
        bool all = true;
        for (int c = c_lo; c <= c_hi; ++c) all = all && ((have >> (NMB * c)) & kAll) != 0;
        if (all) break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit || lds_ld(&s.abort)) {
          lds_st(&s.abort, 1);
          if (lane == 0) atomicOr(a.err, kErrWatchdog);
          return false;
        }
      }
      // row-group form: lane 16 tr + cq sums rows tr + 4 j at columns 4 cq .. + 3
      const int tr = lane >> 4, cq = lane & 15;
      f32x4 v[TP / 4];
#pragma unroll
      for (int k = 0; k < TP / 4; ++k) v[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
      for (int c = c_lo; c <= c_hi; ++c) {
        const int k = ((have >> (NMB * c)) & 1ull) ? 0 : 1;
#pragma unroll
        for (int j = 0; j < TP / 4; ++j) v[j] += *(const f32x4*)&s.mb[c][k][tr + 4 * j][cq * 4];
      }
      for (int c = c_lo; c <= c_hi; ++c) {
        const int k = ((have >> (NMB * c)) & 1ull) ? 0 : 1;
        if (lane == 0) lds_st(&s.tag[c][k], 0);
      }
      const int off = (tm * cm + rank) * TP * 64 * 4 + (tr * 64 + cq * 4) * 4;
#pragma unroll
      for (int j = 0; j < TP / 4; ++j) st16(part, off + j * 4 * 64 * 4, v[j]);
    }
    // contributions: lane i counts this block's (tile, matrix) pairs of tile tau0 + i
    const int tm1 = tm0 + ntm - 1;
    const int tau0 = tm0 / nm, tau1 = tm1 / nm;
    stores_done();
    for (int tau = tau0 + lane; tau <= tau1; tau += 64) {
      int cnt = 0;
      for (int m = 0; m < nm; ++m) {
        const int tm = tau * nm + m;
        if (tm >= tm0 && tm <= tm1) ++cnt;
      }
      __hip_atomic_fetch_add(tk + (size_t)tau * kTicketStride, (unsigned)cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  return true;
}

template <int T>
__device__ __forceinline__ bool svc_own(const StepArgs& a, BlockState<T>& s, int q, int lane, bool ok) {
  constexpr int TP = TPad<T>::value;
  const int l = q >> 2, ph = q & 3;
  const int nm = ph == 2 ? 2 : 1;
  const int tm0 = uniform(s.plan.kp[ph][0]), ntm = uniform(s.plan.kp[ph][1]);
  const int own0 = uniform(s.plan.kp[ph][2]), nown = uniform(s.plan.kp[ph][3]);
  constexpr int G = RG<T>::G;
  constexpr int NPRE = Big<T>::value ? 1 : 2;  // owned tiles whose residual rows are loaded at the phase start
  f32x4 rg[G], xo[NPRE][G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    rg[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NPRE; ++i) xo[i][k] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  // the row factors need every tile of the phase input (its sums of squares)
  if (!wait_ge(a, s, &s.rel, q + 1)) return false;
  if (nown > 0) {
    if (ph == 0 || ph == 2) {
      float r[T];
      rnorm_rows<T>(a, ph == 0 ? 2 * l : 2 * l + 1, lane, r);
      const int tr = lane >> 4;
#pragma unroll
      for (int k = 0; k < G; ++k) {
        float rk = 0.0f;
#pragma unroll
        for (int t = 0; t < T; ++t)
          if (t == tr + 4 * k) rk = r[t];
        rg[k] = (f32x4){rk, rk, rk, rk};
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPRE; ++i)
        if (i < nown) load_rows<T>(a.x, a.H, own0 + i, lane, xo[i]);
    }
  }
  if (!ok) return ok;
  unsigned* tk = a.tickets + ((size_t)l * 4 + ph) * kTicketTiles * kTicketStride;
  // owned tiles: wait for all contributions, then the epilogue
  for (int o = 0; o < nown; ++o) {
    const int tau = own0 + o;
    const uint32_t oc = uniform((uint32_t)s.plan.oc[ph][o][0] | ((uint32_t)s.plan.oc[ph][o][1] << 8));
    const int n0 = oc & 255, n1 = oc >> 8;
    const int expect = n0 + n1;
    unsigned spins = 0;
    while ((int)sld1(tk + (size_t)tau * kTicketStride) < expect) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit || lds_ld(&s.abort)) {
        lds_st(&s.abort, 1);
        if (lane == 0) atomicOr(a.err, kErrWatchdog);
        return false;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    f32x4 xt[G];
    if (o < NPRE) {
#pragma unroll
      for (int k = 0; k < G; ++k) xt[k] = o == 0 ? xo[0][k] : xo[NPRE - 1][k];
    } else if (ph == 1 || ph == 3) {  // more owned tiles than prefetched (small grids)
      load_rows<T>(a.x, a.H, tau, lane, xt);
    } else {
#pragma unroll
      for (int k = 0; k < G; ++k) xt[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    svc_epilogue<T>(a, q, uniform(tau), n0, n1, lane, rg, xt, s.stage);
  }
  // the owned tiles' outputs are complete: count them for the watchers
  if (nown > 0) {
    stores_done();
    if (lane == 0)
      __hip_atomic_fetch_add(a.rdy + ((size_t)(q + 1) * kRdySlots + blockIdx.x % kRdySlots) * kRdyStride, (unsigned)nown,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

template <int T>
__device__ __forceinline__ void svc_lm_prep(const StepArgs& a, int lane, const float (&rt)[T]) {
  const int nc = a.H / 64;
  const int t = lane & 15, kq = lane >> 4;
  // one set of fragments per 16 rows
#pragma unroll
  for (int h = 0; h < (Big<T>::value ? 2 : 1); ++h) {
    const int row = 16 * h + t;
    float r = 0.0f;
#pragma unroll
    for (int i = 0; i < T; ++i)
      if (row == i) r = rt[i] * a.lm_pre;
    const int tt = row < a.T ? row : 0;  // every lane loads an in-range value
    _Float16* frag = a.frag + h * a.frag_half;
    for (int c = blockIdx.x; c < nc; c += gridDim.x) {
      float* o = (float*)(frag + ((size_t)c * 64 + lane) * 32);
      float xr[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) xr[e] = ld_coh(a.x + (size_t)tt * a.H + 64 * c + 16 * kq + e);
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float x0 = row < a.T ? r * xr[e] : 0.0f, x1 = row < a.T ? r * xr[e + 1] : 0.0f;
        const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
        const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
        st_coh(o + e / 2, __builtin_bit_cast(float, (h2){h0, h1}));
        st_coh(o + 8 + e / 2, __builtin_bit_cast(float, (h2){l0, l1}));
      }
    }
  }
}

// The contributions of the block, phase after phase.
template <int T>
__device__ __forceinline__ void contrib_wave(const StepArgs& a, BlockState<T>& s, int lane) {
  bool ok = true;
  for (int q = 0; q < 4 * a.L && ok; ++q) ok = svc_contrib<T>(a, s, q, lane, ok);
}

// The epilogues of the block's tiles, phase after phase; then lm_prep and the
// step's one grid barrier.
template <int T>
__device__ __forceinline__ void owner_wave(const StepArgs& a, BlockState<T>& s, int lane) {
  svc_prep<T>(a, lane, s.stage);
  bool ok = true;
  for (int q = 0; q < 4 * a.L && ok; ++q) ok = svc_own<T>(a, s, q, lane, ok);
  // lm_prep needs the final residual: every tile of the last phase
  if (!ok || !wait_ge(a, s, &s.rel, 4 * a.L + 1)) return;
  float r[T];
  rnorm_rows<T>(a, 2 * a.L, lane, r);
  svc_lm_prep<T>(a, lane, r);
  // the lm phase rewrites the accept lengths that the Gated DeltaNet jobs read
  if (!wait_ge(a, s, &s.gdn_done, 1)) return;
  // the one grid barrier of the step: every block's hidden fragments are in
  svc_barrier<T>(a, s, 0, 4 * a.L, lane, ok, 4 * a.L + 2);
}

// Opens the phases of the block in order: phase q (and, as q = 4L, lm_prep)
// opens once the producer of its input has finished every tile.  Block 0's
// watcher is the only reader of the finished-tile counters: when a producer
// phase is complete it writes the number of open phases into every block's
// own line, which that block's watcher alone polls.  (Many readers polling one
// line slow down its readers and its writers alike.)
template <int T>
__device__ __forceinline__ void watch_wave(const StepArgs& a, BlockState<T>& s, int lane) {
  const int qn = 4 * a.L;
  unsigned spins = 0;
  if (blockIdx.x == 0) {
    for (int q = 0; q <= qn; ++q) {
      const int need = q == 0 || q == qn ? a.H / 64 : line_of(a, q & 3).K / 64;
      const unsigned* c = a.rdy + (size_t)q * kRdySlots * kRdyStride;
      while (true) {
        static_assert(kRdySlots == 8 && kRdyStride == 32, "sld_sum8 reads 8 words 128 B apart");
        const unsigned n = sld_sum8(c);
        if ((int)n >= need) break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit / 8 || lds_ld(&s.abort)) {
          lds_st(&s.abort, 1);
          if (lane == 0) atomicOr(a.err, kErrWatchdog);
          return;
        }
      }
      if (lane == 0 && q + 1 < kMaxStamps) a.stamps[q + 1] = wall_clock64();
      for (int b = lane; b < (int)gridDim.x; b += 64)
        __hip_atomic_store(a.open + (size_t)b * kRdyStride, (unsigned)(q + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) lds_st(&s.rel, q + 1);
    }
  } else {
    const unsigned* mine = a.open + (size_t)blockIdx.x * kRdyStride;
    int rel = 0;
    while (rel <= qn) {
      const int v = (int)sld1(mine);
      if (v > rel) {
        rel = v;
        if (lane == 0) lds_st(&s.rel, rel);
        continue;
      }
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit / 8 || lds_ld(&s.abort)) {
        lds_st(&s.abort, 1);
        if (lane == 0) atomicOr(a.err, kErrWatchdog);
        return;
      }
    }
  }
}

// ------------------------------------------------------------ attention items
// Split-K flash decoding of the full-attention layers beside the layer
// pipeline, like the GDN jobs (the outputs are not fed back).  Item (layer i,
// agent g, KV head h, split s) covers positions [s chunk, min(L_g, (s + 1)
// chunk)) of the agent's cache (L_g = cached positions + the agent's n_g new
// rows, whose k and v are already in the cache), for the agent's n_g rows x
// Hq/Hkv query heads of KV head h (one block of 16 query columns; row r of
// the agent sees positions up to ctx + r).  Its partial goes to the
// workspace, and the last split of (i, g, h) to finish merges all of them
// and applies the output gate.  The tile arithmetic is that of the
// standalone attention launches (mk_attn.h).
constexpr int kAttnPartFloats = 16 * 128 + 16 * 2;

template <bool Q8>
__device__ __forceinline__ void attn_item(const StepArgs& a, int i, int j, int lane_in) {
  // lane-dependent addresses are rebuilt per item: hoisted out of the item
  // loop they stay live through the tile loop and spill
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  int g = 0;
  while (j >= a.attn_item0[g + 1]) ++g;
  g = uniform(g);
  const int ns = uniform(a.attn_nsplit[g]);
  const int per = uniform(a.attn_item0[a.G]);
  const int jg = uniform(a.attn_item0[g]);
  const int loc = j - jg;
  const int h = loc / ns, s = loc - h * ns;
  const int r0 = uniform(a.gs[g]), ng = uniform(a.gs[g + 1]) - r0;
  const int ctx = uniform(a.attn_ctx[g]), Lg = ctx + ng;
  const int p0 = s * a.attn_chunk, p1 = min(Lg, p0 + a.attn_chunk);
  const int gqa = a.attn_gqa, NQ = ng * gqa, Hq = a.attn_Hq;
  const int col = lane & 15, grp = lane >> 4;
  const bool valid = col < NQ;
  const int row = r0 + (valid ? col / gqa : 0), hq = h * gqa + (valid ? col % gqa : 0);
  const int lim = valid ? min(ctx + col / gqa + 1, p1) : 0;  // positions below lim are visible to this column
  // this lane's query column, scaled and split into fp16 hi + lo
  attn::u4 qh[4], ql[4];
  const float* qr = a.attn_q + (((size_t)i * a.T + row) * Hq + hq) * 128 + 8 * grp;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float4 u0 = make_float4(0.f, 0.f, 0.f, 0.f), u1 = u0;
    if (valid) {
      u0 = *(const float4*)(qr + 32 * m);
      u1 = *(const float4*)(qr + 32 * m + 4);
    }
    const float q = a.attn_qscale;
    const float x[8] = {u0.x * q, u0.y * q, u0.z * q, u0.w * q, u1.x * q, u1.y * q, u1.z * q, u1.w * q};
    attn::split_f16(x, qh[m], ql[m]);
  }
  const size_t gh = ((size_t)i * a.G + g) * a.attn_Hkv + h;
  attn::KVHead kv = {};
  kv.cap = a.attn_cap;
  if constexpr (Q8) {
    kv.K8 = a.attn_k8 + gh * kv.cap * 128;
    kv.KS = a.attn_ks + gh * kv.cap * 4;
    kv.V8 = a.attn_v8 + gh * 128 * kv.cap;
    kv.VS = a.attn_vs + gh * (kv.cap / 32) * 128;
  } else {
    kv.K = a.attn_k + gh * kv.cap * 128;
    kv.V = a.attn_v + gh * 128 * kv.cap;
  }
  attn::f4 acc[8];
  float mrow = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = attn::f4{0.f, 0.f, 0.f, 0.f};
  for (int t0 = p0; t0 < p1; t0 += attn::kTile) {
    attn::KVTile x;
    attn::load_tile<Q8>(kv, t0, Lg, col, grp, x);
    attn::tile_update<Q8>(x, t0, Lg, lim, grp, qh, ql, acc, mrow, lsum);
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  // the item's partial: lane (col, grp) holds dims 16 db + 4 grp .. + 3 of column col
  float* po = a.attn_part + ((size_t)i * per + j) * kAttnPartFloats;
#pragma unroll
  for (int db = 0; db < 8; ++db) st16(po, (col * 128 + 16 * db + 4 * grp) * 4, acc[db]);
  if (grp == 0) {
    st_coh(po + 2048 + 2 * col, mrow);
    st_coh(po + 2048 + 2 * col + 1, lsum);
  }
  int last = 0;
  if (lane == 0) last = ticket_add(a.attn_ticket + gh * 16) == (unsigned)(ns - 1);
  if (!__shfl(last, 0, 64)) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // merge the splits: lane (col, grp) takes dims 32 grp .. 32 grp + 31 of column col
  const float* pb = a.attn_part + ((size_t)i * per + jg + (size_t)h * ns) * kAttnPartFloats;
  float m = -INFINITY, l = 0.f;
  attn::f4 y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = attn::f4{0.f, 0.f, 0.f, 0.f};
  for (int s2 = 0; s2 < ns; ++s2) {
    const float* ps = pb + (size_t)s2 * kAttnPartFloats;
    const float ms = ld_coh(ps + 2048 + 2 * col), ls = ld_coh(ps + 2048 + 2 * col + 1);
    const float mn = fmaxf(m, ms);
    if (mn == -INFINITY) continue;
    const float ao = exp2f(m - mn), as = exp2f(ms - mn);
    l = l * ao + ls * as;
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = y[k] * ao + ld16(ps, (col * 128 + 32 * grp + 4 * k) * 4) * as;
    m = mn;
  }
  if (!valid) return;
  const size_t ob = (((size_t)i * a.T + row) * Hq + hq) * 128 + 32 * grp;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    attn::f4 v = y[k] / l;
    if (a.attn_gate) {
      const float4 gt = *(const float4*)(a.attn_gate + ob + 4 * k);
      v[0] *= 1.f / (1.f + expf(-gt.x));
      v[1] *= 1.f / (1.f + expf(-gt.y));
      v[2] *= 1.f / (1.f + expf(-gt.z));
      v[3] *= 1.f / (1.f + expf(-gt.w));
    }
    *(attn::f4*)(a.attn_o + ob + 4 * k) = v;
  }
}

// WITH: the kernel instance that runs attention items (either cache
// format).  The instance for steps without attention carries none of their
// code: their register demand (and the q8_0 items' spilled registers) would
// otherwise cost every step.
template <bool WITH>
__device__ __forceinline__ void attn_items(const StepArgs& a, int lane) {
  if constexpr (WITH) {
    if (a.n_attn <= 0) return;
    const int per = uniform(a.attn_item0[a.G]);
    const long total = (long)a.n_attn * per;
    if (a.attn_q8)
      for (long it = blockIdx.x; it < total; it += gridDim.x) attn_item<true>(a, (int)(it / per), (int)(it % per), lane);
    else
      for (long it = blockIdx.x; it < total; it += gridDim.x) attn_item<false>(a, (int)(it / per), (int)(it % per), lane);
  }
}

// The block's share of every GDN layer's half-head jobs, in layer order.
// Nothing in the step consumes their outputs, so they run beside the layer
// pipeline instead of inside one of its phases; the block's last barrier
// waits for them (see service_wave).
// Jobs are numbered over the whole step (GDN layer i, job j: i * nj + j) and
// dealt to the blocks round-robin, so that the blocks share them evenly
// even when a layer has fewer jobs than there are blocks (one agent: 64 jobs
// per layer for 256 blocks).  The GDN wave shares its SIMD with a compute
// wave, so an uneven share would slow that block's streaming.
__device__ __forceinline__ void gdn_wave(const StepArgs& a, int lane) {
  if (a.n_agents <= 0) return;
  const long nj = (long)a.n_agents * kGdnHeadsPerLayer * 2;
  const long nb = gridDim.x;
  long i = 0;  // GDN layers seen
  for (int l = 0; l < a.L; ++l) {
    if (!layer_is_gdn(a, l)) continue;
    long j = ((long)blockIdx.x - i * nj) % nb;
    if (j < 0) j += nb;
    for (; j < nj; j += nb) gdn_job(a, l, j, lane);
    ++i;
  }
}

// The lm_head stream over the final hidden rows (fragments written by
// lm_prep), then the argmax and the accept compare in the last block.  The
// ring area, free after the last GEMV phase, holds the LDS-staged stream's
// three stages (hidden size 5120 or 512) or the other stream's cross-wave
// sums.
__device__ __forceinline__ void lm_phase(const StepArgs& a, uint8_t* ring) {
  __shared__ int fin[16];
  __shared__ int tops[32];  // the argmax of every row
  // one stream over the vocabulary per 16 rows
  const int npass = (a.T + 15) / 16;
  bool last = false;
  for (int h = 0; h < npass; ++h) {
    LmStream ls;
    ls.W = a.lm;
    ls.frag = a.frag + h * a.frag_half;
    ls.V = a.V;
    ls.H = a.H;
    ls.val = a.lm_val + (size_t)h * gridDim.x * 16;
    ls.idx = a.lm_idx + (size_t)h * gridDim.x * 16;
    ls.ticket = a.lm_ticket + h * kRdyStride;
    ls.logits = nullptr;
    ls.logits_T = 0;
    static_assert(kWavesPerBlock == 8, "the staged stream runs on 8 waves");
    if (a.H == 5120)
      last = lm_stream_staged<3, 10>(ls, ring, fin);
    else if (a.H == 512)
      last = lm_stream_staged<3, 1>(ls, ring, fin);
    else
      last = lm_stream<kWavesPerBlock>(ls, (float (*)[64][16])ring, fin);
    if (last && h + 1 < npass) {
      // the last block of an earlier stream hands its rows to the last block of the final one
      if (threadIdx.x < 16) __hip_atomic_store(a.out + kOutTop + 16 * h + threadIdx.x, fin[threadIdx.x],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      stores_done();
      __syncthreads();
      if (threadIdx.x == 0) ticket_add((unsigned*)(a.out + kOutPass));
    }
  }
  if (!last) return;
  if (threadIdx.x == 0 && npass > 1) {
    unsigned spins = 0;
    while (__hip_atomic_load(a.out + kOutPass, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < npass - 1) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        atomicOr(a.err, kErrWatchdog);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  __syncthreads();
  if (threadIdx.x < 16 * npass)
    tops[threadIdx.x] = (int)threadIdx.x >= 16 * (npass - 1)
                            ? fin[threadIdx.x - 16 * (npass - 1)]
                            : __hip_atomic_load(a.out + kOutTop + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int t = 0; t < a.T; ++t) a.out[kOutTop + t] = tops[t];
    for (int g = 0; g < a.G; ++g) {
      const int r = a.gs[g], n = a.gs[g + 1] - a.gs[g];
      const int32_t* dr = a.drafts + (r - g);
      int k = 0;
      while (k < n - 1 && tops[r + k] >= 0 && dr[k] == tops[r + k]) ++k;
      a.out[kOutNacc + g] = k;
      for (int i = 0; i < n; ++i) a.out[kOutTok + r + i] = i < k ? dr[i] : (i == k ? tops[r + k] : -1);
      if (g < a.n_agents) {
        a.nacc[g][0] = k;      // replayed by the next step
        a.nacc[g][1] ^= 1;     // this step's rows are in the other ring half
      }
    }
  }
}

// ------------------------------------------------------------ the kernel
template <int T, bool ATTN>
__global__ __launch_bounds__(kBlock) void k_decode_step(StepArgs a) {
  __shared__ BlockState<T> s;
  const int lane = threadIdx.x & 63;
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The weight table and block plans in the workspace must be this stack's
  // (written before the launch; every block reads the same tag, so either
  // every block runs or none does).
  if (threadIdx.x == 0) s.abort = *a.ws_tag != a.tag;
  __syncthreads();
  if (s.abort) {
    if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(a.err, kErrTables);
    return;
  }
  if (threadIdx.x < BlockState<T>::NMB * kCompute) (&s.tag[0][0])[threadIdx.x] = 0;
  if (threadIdx.x < kCompute) s.done[threadIdx.x] = 0;
  // the weight table is written before the launch: plain loads are safe
  for (int i = threadIdx.x; i < a.L * 5; i += kBlock) s.wt[i / 5][i % 5] = a.layers[i / 5].w[i % 5];
  for (int i = threadIdx.x; i < kPlanWords / 4; i += kBlock)
    ((u32x4*)&s.plan)[i] = ((const u32x4*)(a.plans + blockIdx.x))[i];
  if (threadIdx.x == 0) {
    s.rel = 0;
    s.abort = 0;
    s.gdn_done = 0;
    for (int i = 0; i < (int)sizeof(s.stage) / 4; ++i) ((int*)s.stage)[i] = 0;
    if (blockIdx.x == 0) a.stamps[0] = wall_clock64();
  }
  __syncthreads();
  if (wib < kCompute) {
    compute_wave<T>(a, s, wib, lane);
  } else if (wib == kServiceWave) {
    contrib_wave<T>(a, s, lane);
  } else if (wib == kOwnerWave) {
    owner_wave<T>(a, s, lane);
  } else if (wib == kWatchWave) {
    watch_wave<T>(a, s, lane);
  } else {
    gdn_wave(a, lane);
    attn_items<ATTN>(a, lane);
    stores_done();
    if (lane == 0) lds_st(&s.gdn_done, 1);
  }
  // every wave of the block takes part in the lm phase once lm_prep is done
  if (!wait_ge(a, s, &s.rel, 4 * a.L + 2)) return;
  static_assert(sizeof(s.ring) >= sizeof(float) * kWavesPerBlock * 64 * 16, "lm reduction does not fit the ring");
  static_assert(sizeof(s.ring) >= 3 * kLmStageBytes, "the lm stages do not fit the ring");
  lm_phase(a, &s.ring[0][0]);
  if (blockIdx.x == 0 && threadIdx.x == 0) a.stamps[kMaxStamps - 1] = wall_clock64();
}

// ------------------------------------------------------------ host side
typedef void (*StepKernel)(StepArgs);

template <int T>
static StepKernel kernel_for(bool attn) {
  return attn ? k_decode_step<T, true> : k_decode_step<T, false>;
}

// attn: the instance that runs attention items.
static StepKernel step_kernel(int T, bool attn = false) {
  switch (T) {
    case 1: return kernel_for<1>(attn);
    case 2: return kernel_for<2>(attn);
    case 3: return kernel_for<3>(attn);
    case 4: return kernel_for<4>(attn);
    case 5: return kernel_for<5>(attn);
    case 6: return kernel_for<6>(attn);
    case 7: return kernel_for<7>(attn);
    case 8: return kernel_for<8>(attn);
    case 9: return kernel_for<9>(attn);
    case 10: return kernel_for<10>(attn);
    case 11: return kernel_for<11>(attn);
    case 12: return kernel_for<12>(attn);
    case 13: return kernel_for<13>(attn);
    case 14: return kernel_for<14>(attn);
    case 15: return kernel_for<15>(attn);
    case 16: return kernel_for<16>(attn);
    case 17: return kernel_for<17>(attn);
    case 18: return kernel_for<18>(attn);
    case 19: return kernel_for<19>(attn);
    case 20: return kernel_for<20>(attn);
    case 21: return kernel_for<21>(attn);
    case 22: return kernel_for<22>(attn);
    case 23: return kernel_for<23>(attn);
    case 24: return kernel_for<24>(attn);
    default: return nullptr;
  }
}

// ---------------------------------------------------------------------------
// Streaming GEMV: the standalone T-row GEMV and FFN (T <= 16) on the step's
// engines and activation records (the MK_PATH_STEP path of mk_qgemv_rows_ex,
// and mk_ffn_rows).  The records are written by the step's own epilogue
// quantizer (store_q8) and every unit goes through the engine the step uses
// for T rows, so the integer sums of those engines and the record layout
// can also be checked exactly outside the persistent launch.
//
// A stage's units form a line, tile-major over (tile, matrix) pairs.  Blocks
// of 4 compute waves and 1 service wave, one block per CU; compute wave gw of
// Wc takes units [U gw / Wc, U (gw + 1) / Wc) and streams them through a
// private 2-slot LDS ring (each slot: the unit and the record of its
// superblock, both by LDS-DMA), so the next unit's loads are in flight during
// the current unit's arithmetic.  The sums of each (tile, matrix) go to one of
// the wave's two LDS mailboxes; the service wave adds the block's mailboxes in
// wave order, stores one partial per (tile, matrix, block) and counts it on
// the tile's ticket, and the block whose count completes a tile adds the
// tile's partials in block order and runs the epilogue: y, or SiLU(gate) * up
// quantized into the next stage's record.  No block waits for another, so
// the launch needs no co-residency.

// Activation record part of the 64-column tile blockIdx.x of x [T][K]; block
// 0 also clears the nzero ticket words of the stages that follow.
template <int T>
__global__ __launch_bounds__(64) void k_engine_records(const float* __restrict__ x, int K, uint8_t* rec,
                                                       unsigned* zero, int nzero) {
  __shared__ uint8_t stage[kStageBytes] __attribute__((aligned(16)));
  const int lane = threadIdx.x, tau = blockIdx.x;
  if (tau == 0)
    for (int i = lane; i < nzero; i += 64) zero[i] = 0u;
  // rows >= TPad stay zero in the stage, as in the step
  for (int i = lane; i < kStageBytes / 4; i += 64) ((int*)stage)[i] = 0;
  __syncthreads();
  f32x4 v[RG<T>::G];
  load_rows<T>(x, K, tau, lane, v);
  store_q8<T>(rec, tau, lane, v, stage);
}

struct StreamArgs {
  const uint8_t* W0;
  const uint8_t* W1;   // the second matrix of a pair (gate/up), else W0
  const uint8_t* rec;  // input records [nsb][kActBytes]
  float* part;         // [(tile, matrix)][cmax][TP][64]
  unsigned* tickets;   // [ntiles], kTicketStride words apart, zero at launch
  float* y;            // epi 0: y [T][N]; epi 1: h [T][N] or null
  uint8_t* rec_out;    // epi 1: the records of h
  int nsb, ntiles, mshift, U, cmax, N, epi;  // mshift: log2 of the matrices per tile (0 or 1)
};

constexpr int kStreamThreads = 64 * (kCompute + 1);

template <int T>
struct StreamState {
  uint8_t ring[kCompute][kSlots * kSlotBytes] __attribute__((aligned(16)));
  float mb[kCompute][2][TPad<T>::value][kMbRow] __attribute__((aligned(16)));  // [t][row of the tile]
  uint8_t stage[kStageBytes] __attribute__((aligned(16)));
  int tag[kCompute][2];  // (tile, matrix) + 1 of a full mailbox, 0 when free
  int abort;
};

// The part holding unit u when a line of U units is cut into n parts, part p
// being [U p / n, U (p + 1) / n).
__device__ __forceinline__ int part_of(long u, int n, long U) { return (int)(((u + 1) * n - 1) / U); }

// Blocks contributing to (tile, matrix) tm, and the first of them.
__device__ __forceinline__ int stream_first_block(const StreamArgs& a, int tm) {
  return part_of((long)tm * a.nsb, (int)gridDim.x, a.U);
}
__device__ __forceinline__ int stream_blocks(const StreamArgs& a, int tm) {
  return part_of((long)tm * a.nsb + a.nsb - 1, (int)gridDim.x, a.U) - stream_first_block(a, tm) + 1;
}

// Starts the weight loads of unit (tm, b) into the slot at LDS address lds,
// then (separately) the loads of the record of its superblock.
__device__ __forceinline__ void stream_issue_w(const StreamArgs& a, uint32_t lds, int tm, int b, int lane) {
  const size_t w0 = opaque((size_t)a.W0), w1 = opaque((size_t)a.W1);
  const uint8_t* W = (const uint8_t*)((tm & ((1 << a.mshift) - 1)) ? w1 : w0);
  dma<9, false>(lds, W + ((size_t)(tm >> a.mshift) * a.nsb + b) * kUnitBytes + lane * 16);
}
__device__ __forceinline__ void stream_issue_a(const StreamArgs& a, uint32_t lds, int b, int lane) {
  dma<5, false>(lds + kUnitBytes, a.rec + (size_t)b * kActBytes + lane * 16);
}

// The wave's sums of (tile, matrix) tm into mailbox nflush % 2, as [t][row].
template <int T>
__device__ __forceinline__ void stream_flush(StreamState<T>& s, int c, int lane, int tm, int nflush, float (&acc)[T],
                                             f32x4 (&macc)[4], bool& ok) {
  const int slot = nflush & 1;
  unsigned spins = 0;
  while (ok && lds_ld(&s.tag[c][slot]) != 0) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpinLimit || lds_ld(&s.abort)) {
      lds_st(&s.abort, 1);
      ok = false;
    }
  }
  if (!ok) return;
  if constexpr (UseMfma<T>::value) {
    if constexpr (PackMfma<T>::value) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) macc[nb][i] += __shfl_xor(macc[nb][i], 32, 64);
    }
    const int q = lane >> 4, n = lane & 15;
    if (4 * q < TPad<T>::value)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s.mb[c][slot][4 * q + i][16 * nb + n] = macc[nb][i];
  } else {
#pragma unroll
    for (int t = 0; t < T; ++t) s.mb[c][slot][t][lane] = acc[t];
  }
  if (lane == 0) lds_st(&s.tag[c][slot], tm + 1);
}

template <int T>
__device__ __forceinline__ void stream_compute(const StreamArgs& a, StreamState<T>& s, int c, int lane) {
  const int Wc = (int)gridDim.x * kCompute, gw = (int)blockIdx.x * kCompute + c;
  const long U = a.U;
  const int u0 = (int)(U * gw / Wc), u1 = (int)(U * (gw + 1) / Wc);
  if (u0 >= u1) return;
  const int nsb = a.nsb;
  const uint32_t l[2] = {(uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&s.ring[c][0],
                         (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&s.ring[c][kSlotBytes]};
  int itm = u0 / nsb, ib = u0 - itm * nsb;  // the next unit to load
  int ctm = itm;                            // (tile, matrix) of the unit consumed next
  int cb = ib;
  stream_issue_w(a, l[0], itm, ib, lane);
  stream_issue_a(a, l[0], ib, lane);
  if (++ib == nsb) ib = 0, ++itm;
  if (u0 + 1 < u1) {
    stream_issue_w(a, l[1], itm, ib, lane);
    stream_issue_a(a, l[1], ib, lane);
    if (++ib == nsb) ib = 0, ++itm;
  }
  float acc[T];
  f32x4 macc[4];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) macc[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  int open = ctm, nflush = 0;
  bool ok = true;
  for (int u = u0; u < u1 && ok; ++u) {
    const int k = (u - u0) & 1;
    // this slot's 14 loads were issued before the other slot's
    if (u + 1 < u1)
      wait_ops(14);
    else
      wait_ops(0);
    if (ctm != open) {
      stream_flush<T>(s, c, lane, open, nflush++, acc, macc, ok);
      open = ctm;
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) macc[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    lds_u8* sl = as_lds(&s.ring[c][k * kSlotBytes]);
    const bool refill = u + 2 < u1;
    // The matrix-core engines copy the unit's weights into registers and
    // refill the slot's weight region before their arithmetic (so those loads
    // have two units' arithmetic to arrive); the record region, which the
    // arithmetic reads, is refilled after it.  Loads complete in issue order
    // (weights of u + 2, record of u + 2, weights of u + 3, ...), so waiting
    // for all but the next unit's 14 loads still means this slot is in.
    if constexpr (!UseMfma<T>::value) {
      slot_dot4<T>(sl, lane, acc);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (refill) stream_issue_w(a, l[k], itm, ib, lane);
    } else if constexpr (PackMfma<T>::value) {
      WregP xw;
      read_w_pk(sl, lane, xw);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (refill) stream_issue_w(a, l[k], itm, ib, lane);
      slot_mfma_pk(xw, sl, lane, macc);
    } else {
      WregM xw;
      read_w_mfma(sl, lane, xw);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (refill) stream_issue_w(a, l[k], itm, ib, lane);
      slot_mfma(xw, sl, lane, macc);
    }
    // every LDS read of the record has completed before it is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (refill) {
      stream_issue_a(a, l[k], ib, lane);
      if (++ib == nsb) ib = 0, ++itm;
    }
    if (++cb == nsb) cb = 0, ++ctm;
  }
  if (ok) stream_flush<T>(s, c, lane, open, nflush, acc, macc, ok);
  wait_ops(0);  // no load outlives the wave
}

// The epilogue of tile tau: its partials added in block order (row-group
// form: lane 16 tr + cq holds rows tr + 4 k at columns 4 cq .. + 3).
template <int T>
__device__ __forceinline__ void stream_epilogue(const StreamArgs& a, StreamState<T>& s, int tau, int lane) {
  constexpr int TP = TPad<T>::value, G = RG<T>::G;
  const int tr = lane >> 4, cq = lane & 15;
  const int nm = 1 << a.mshift;
  f32x4 v[2][G];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int k = 0; k < G; ++k) v[m][k] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int m = 0; m < nm; ++m) {
    const int tm = (tau << a.mshift) + m;
    const int n = stream_blocks(a, tm);
    const float* pb = a.part + (size_t)tm * a.cmax * TP * 64;
    for (int r0 = 0; r0 < n; r0 += 4) {
      f32x4 t[4][G];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + i < n ? r0 + i : n - 1;  // in-range address; extra values are not added
#pragma unroll
        for (int k = 0; k < G; ++k) t[i][k] = ld16(pb, ((r * TP + tr + 4 * k) * 64 + cq * 4) * 4);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (r0 + i >= n) break;
#pragma unroll
        for (int k = 0; k < G; ++k) {
          if (m == 0)
            v[0][k] += t[i][k];
          else
            v[1][k] += t[i][k];
        }
      }
    }
  }
  // rows >= T of a partial are not results (the dot-product engine leaves them unset)
#pragma unroll
  for (int k = 0; k < G; ++k)
    if (tr + 4 * k >= T) v[0][k] = v[1][k] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int col = tau * 64 + cq * 4;
  if (a.epi == 0) {
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int t = tr + 4 * k;
      if (t >= T) continue;
      if (col + 3 < a.N) {
        st16(a.y, (t * a.N + col) * 4, v[0][k]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (col + i < a.N) a.y[(size_t)t * a.N + col + i] = v[0][k][i];
      }
    }
    return;
  }
  f32x4 h[G];
#pragma unroll
  for (int k = 0; k < G; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = v[0][k][i], u = v[1][k][i];
      h[k][i] = g * u / (1.0f + expf(-g));
    }
  if (a.y)
#pragma unroll
    for (int k = 0; k < G; ++k)
      if (tr + 4 * k < T) st16(a.y, ((tr + 4 * k) * a.N + col) * 4, h[k]);
  store_q8<T>(a.rec_out, tau, lane, h, s.stage);
}

template <int T>
__device__ __forceinline__ void stream_service(const StreamArgs& a, StreamState<T>& s, int lane) {
  constexpr int TP = TPad<T>::value;
  const int nblk = (int)gridDim.x, Wc = nblk * kCompute, blk = (int)blockIdx.x;
  const long U = a.U;
  // every block holds units (the grid has at most U blocks), so every block
  // between the first and the last of a (tile, matrix) contributes to it
  const int ub0 = (int)(U * blk / nblk), ub1 = (int)(U * (blk + 1) / nblk);
  if (ub0 >= ub1) return;
  const int nsb = a.nsb;
  const int tr = lane >> 4, cq = lane & 15;
  for (int tm = ub0 / nsb; tm <= (ub1 - 1) / nsb; ++tm) {
    // the block's waves holding units of tm (a wave's stretch may be empty
    // when the line has fewer units than the grid has compute waves)
    unsigned cmask = 0;
    for (int c = 0; c < kCompute; ++c) {
      const long gw = (long)blk * kCompute + c;
      const long w0 = U * gw / Wc, w1 = U * (gw + 1) / Wc;
      if (max(w0, (long)tm * nsb) < min(w1, (long)(tm + 1) * nsb)) cmask |= 1u << c;
    }
    const int want = tm + 1;
    uint64_t have = 0;
    unsigned spins = 0;
    while (true) {
      const int tg = lane < 2 * kCompute ? lds_ld(&s.tag[lane >> 1][lane & 1]) : 0;
      have = __ballot(tg == want);
      bool all = true;
      for (int c = 0; c < kCompute; ++c)
        if ((cmask >> c) & 1u) all = all && ((have >> (2 * c)) & 3ull) != 0;
      if (all) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit || lds_ld(&s.abort)) {
        lds_st(&s.abort, 1);
        return;
      }
    }
    f32x4 v[TP / 4];
#pragma unroll
    for (int j = 0; j < TP / 4; ++j) v[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < kCompute; ++c) {
      if (!((cmask >> c) & 1u)) continue;
      const int k = ((have >> (2 * c)) & 1ull) ? 0 : 1;
#pragma unroll
      for (int j = 0; j < TP / 4; ++j) v[j] += *(const f32x4*)&s.mb[c][k][tr + 4 * j][cq * 4];
    }
    for (int c = 0; c < kCompute; ++c) {
      if (!((cmask >> c) & 1u)) continue;
      const int k = ((have >> (2 * c)) & 1ull) ? 0 : 1;
      if (lane == 0) lds_st(&s.tag[c][k], 0);
    }
    float* pp = a.part + ((size_t)tm * a.cmax + (blk - stream_first_block(a, tm))) * TP * 64;
#pragma unroll
    for (int j = 0; j < TP / 4; ++j) st16(pp, ((tr + 4 * j) * 64 + cq * 4) * 4, v[j]);
    // count the partial on the tile's ticket; the block completing the tile runs its epilogue
    const int tau = tm >> a.mshift;
    int expect = 0;
    for (int m = 0; m < (1 << a.mshift); ++m) expect += stream_blocks(a, (tau << a.mshift) + m);
    unsigned old = 0;
    if (lane == 0) old = ticket_add(a.tickets + (size_t)tau * kTicketStride);  // after the partial's stores
    old = __shfl(old, 0, 64);
    if ((int)old == expect - 1) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      stream_epilogue<T>(a, s, tau, lane);
    }
  }
}

template <int T>
__global__ __launch_bounds__(kStreamThreads) void k_stream(StreamArgs a) {
  __shared__ StreamState<T> s;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (threadIdx.x < 2 * kCompute) (&s.tag[0][0])[threadIdx.x] = 0;
  if (threadIdx.x == 0) s.abort = 0;
  for (int i = threadIdx.x; i < kStageBytes / 4; i += kStreamThreads) ((int*)s.stage)[i] = 0;
  __syncthreads();
  if (w < kCompute)
    stream_compute<T>(a, s, w, lane);
  else
    stream_service<T>(a, s, lane);
}

// The launch shape of one stage: blocks (at most one per CU, at least one
// unit per compute wave where possible) and the partial slots per (tile,
// matrix): a (tile, matrix) has nsb consecutive units, so it meets at most
// floor((nsb - 1) nblk / U) + 2 blocks.
struct StreamPlan {
  int nblk, ntiles, nsb, nm, U, cmax;
};

static StreamPlan stream_plan(int N, int K, int nm, int cu) {
  StreamPlan p;
  p.ntiles = (N + 63) / 64;
  p.nsb = K / 256;
  p.nm = nm;
  p.U = p.ntiles * nm * p.nsb;
  const int c = cu > 0 ? cu : 256;
  p.nblk = std::max(1, std::min(c, (p.U + kCompute - 1) / kCompute));
  p.cmax = (int)(((long)(p.nsb - 1) * p.nblk) / p.U) + 2;
  return p;
}

static size_t stream_part_bytes(int T, const StreamPlan& p) {
  return (((size_t)p.ntiles * p.nm * p.cmax * ((T + 3) & ~3) * 64 * 4) + 255) & ~(size_t)255;
}

static size_t rec_bytes(int K) { return (((size_t)(K / 256) * kActBytes) + 255) & ~(size_t)255; }
static size_t ticket_bytes(int ntiles) { return (((size_t)ntiles * kTicketStride * 4) + 255) & ~(size_t)255; }

template <int T>
static void launch_stream_t(const StreamPlan& p, const uint8_t* W0, const uint8_t* W1, const uint8_t* rec, float* part,
                            unsigned* tickets, int epi, float* y, uint8_t* rec_out, int N, hipStream_t st) {
  StreamArgs a;
  a.W0 = W0;
  a.W1 = W1 ? W1 : W0;
  a.rec = rec;
  a.part = part;
  a.tickets = tickets;
  a.y = y;
  a.rec_out = rec_out;
  a.nsb = p.nsb;
  a.ntiles = p.ntiles;
  a.mshift = p.nm == 2 ? 1 : 0;
  a.U = p.U;
  a.cmax = p.cmax;
  a.N = N;
  a.epi = epi;
  hipLaunchKernelGGL(k_stream<T>, dim3(p.nblk), dim3(kStreamThreads), 0, st, a);
}

template <int T>
static void launch_records_t(const float* x, int K, uint8_t* rec, unsigned* zero, int nzero, hipStream_t st) {
  hipLaunchKernelGGL(k_engine_records<T>, dim3(K / 64), dim3(64), 0, st, x, K, rec, zero, nzero);
}

#define MK_T_CASES(F, ...)                  \
  switch (T) {                              \
    case 1: F<1>(__VA_ARGS__); break;       \
    case 2: F<2>(__VA_ARGS__); break;       \
    case 3: F<3>(__VA_ARGS__); break;       \
    case 4: F<4>(__VA_ARGS__); break;       \
    case 5: F<5>(__VA_ARGS__); break;       \
    case 6: F<6>(__VA_ARGS__); break;       \
    case 7: F<7>(__VA_ARGS__); break;       \
    case 8: F<8>(__VA_ARGS__); break;       \
    case 9: F<9>(__VA_ARGS__); break;       \
    case 10: F<10>(__VA_ARGS__); break;     \
    case 11: F<11>(__VA_ARGS__); break;     \
    case 12: F<12>(__VA_ARGS__); break;     \
    case 13: F<13>(__VA_ARGS__); break;     \
    case 14: F<14>(__VA_ARGS__); break;     \
    case 15: F<15>(__VA_ARGS__); break;     \
    case 16: F<16>(__VA_ARGS__); break;     \
    default: return hipErrorInvalidValue;   \
  }

// Workspace of the GEMV: x's records, the tickets, the partials.
size_t engine_gemv_workspace(int T, int N, int K, int cu) {
  const StreamPlan p = stream_plan(N, K, 1, cu);
  return rec_bytes(K) + ticket_bytes(p.ntiles) + stream_part_bytes(T, p);
}

hipError_t launch_engine_gemv(const uint8_t* W, int N, int K, const float* x, int T, float* y, uint8_t* ws, int cu,
                              hipStream_t st) {
  const StreamPlan p = stream_plan(N, K, 1, cu);
  uint8_t* rec = ws;
  unsigned* tk = (unsigned*)(ws + rec_bytes(K));
  float* part = (float*)(ws + rec_bytes(K) + ticket_bytes(p.ntiles));
  MK_T_CASES(launch_records_t, x, K, rec, tk, p.ntiles * kTicketStride, st)
  MK_T_CASES(launch_stream_t, p, W, nullptr, rec, part, tk, 0, y, nullptr, N, st)
  return hipGetLastError();
}

// Workspace of the FFN: x's records, h's records, the tickets of both stages,
// the partials of gate/up, then of down.
size_t engine_ffn_workspace(int T, int H, int F, int cu) {
  const StreamPlan pg = stream_plan(F, H, 2, cu), pd = stream_plan(H, F, 1, cu);
  return rec_bytes(H) + rec_bytes(F) + ticket_bytes(pg.ntiles + pd.ntiles) + stream_part_bytes(T, pg) +
         stream_part_bytes(T, pd);
}

hipError_t launch_engine_ffn(const uint8_t* gate, const uint8_t* up, const uint8_t* down, int H, int F, const float* x,
                             int T, float* y, float* h_out, uint8_t* ws, int cu, hipStream_t st) {
  const StreamPlan pg = stream_plan(F, H, 2, cu), pd = stream_plan(H, F, 1, cu);
  uint8_t* rx = ws;
  uint8_t* rh = rx + rec_bytes(H);
  unsigned* tk = (unsigned*)(rh + rec_bytes(F));
  unsigned* tkd = tk + (size_t)pg.ntiles * kTicketStride;
  float* pgu = (float*)((uint8_t*)tk + ticket_bytes(pg.ntiles + pd.ntiles));
  float* pdn = (float*)((uint8_t*)pgu + stream_part_bytes(T, pg));
  MK_T_CASES(launch_records_t, x, H, rx, tk, (pg.ntiles + pd.ntiles) * kTicketStride, st)
  MK_T_CASES(launch_stream_t, pg, gate, up, rx, pgu, tk, 1, h_out, rh, F, st)
  MK_T_CASES(launch_stream_t, pd, down, nullptr, rh, pdn, tkd, 0, y, nullptr, H, st)
  return hipGetLastError();
}
#undef MK_T_CASES

}  // namespace mk

using namespace mk;

struct mk_stack {
  mk_stack_desc d;
  std::vector<LayerW> layers;
  std::vector<mk_deltanet> dn;
  std::vector<uint8_t> gdn_flag;
  int n_gdn_layers = 0;
  int8_t gdn_idx[kMaxLayers];
  uint64_t tag = 0;              // unique per stack; written into a workspace with its tables
  std::vector<BlockPlan> plans;  // for plans_grid blocks
  int plans_grid = -1;
  hipEvent_t ev[2] = {nullptr, nullptr};  // around the last launch (no device memory)
  float last_ms = -1.0f;
  int32_t* hout = nullptr;  // pinned host copy of the output block (allocated at the first step)
};

namespace {

size_t a256(size_t n) { return (n + 255) / 256 * 256; }

// Which stack's weight table and block plans each workspace holds.  A
// workspace is bound to the last stack that ran a step on it; a step by
// another stack uploads its own tables again.  The kernel checks the tag
// written beside the tables, so a workspace that some other call wrote in
// between is caught on the device.
std::mutex g_ws_mu;
std::map<const void*, uint64_t> g_ws_tables;
std::atomic<uint64_t> g_next_tag{1};

struct StepLayout {
  int grid, Wc;
  int cmax[4];
  size_t off_ctrl, n_ctrl;  // zeroed before each launch: barrier, tickets
  size_t off_rdy, off_open, part_half;
  size_t off_plans, off_tag;
  size_t off_out, off_stamps, off_tickets, off_lmticket, off_table, off_act, off_ss, off_part, off_frag, off_lmv,
      off_lmi, total;
  size_t act_layer, act_off[4];
  size_t frag_half;  // lm_head input fragments per 16 rows (fp16 elements)
};

// Compute waves in the order they take a line's remainder units: the waves on
// SIMDs 2 and 3 first (those SIMDs' other waves, the watcher and the owner,
// mostly sleep), then the one beside the GDN wave, last the one beside the
// service wave, which sums and publishes the block's contributions as the
// phase ends.  (Measured on the 64-layer stack: 0.4 to 0.9 % off the step
// against an even spread; handing it to the service wave's neighbour first costs 1.2 %.)
constexpr int kRemainderOrder[kCompute] = {2, 3, 1, 0};

// The split of a line of S units over the grid's Wc compute waves, as
// contiguous ranges in wave order: wave w takes [lo[w], lo[w + 1]).  With at
// least one unit per wave, every wave takes S / Wc units and the S % Wc left
// over go one each to the waves of kRemainderOrder's first entries, spread
// evenly over the blocks; a shorter line gives one unit to each of its first
// S waves.
struct UnitSplit {
  std::vector<long> lo;
  UnitSplit(long S, long Wc) : lo(Wc + 1, S) {
    if (S < Wc) {
      for (long w = 0; w < S; ++w) lo[w] = w;
      return;
    }
    const long nb = Wc / kCompute;
    std::vector<long> n(Wc, S / Wc);
    long r = S % Wc;
    for (int t = 0; t < kCompute && r > 0; ++t) {
      const long k = std::min(r, nb), c = kRemainderOrder[t];
      for (long b = 0; b < nb; ++b) n[b * kCompute + c] += (b + 1) * k / nb - b * k / nb;
      r -= k;
    }
    lo[0] = 0;
    for (long w = 0; w < Wc; ++w) lo[w + 1] = lo[w] + n[w];
  }
  // the wave whose range holds unit p (0 <= p < S)
  long wave_of(long p) const { return (long)(std::upper_bound(lo.begin(), lo.end(), p) - lo.begin()) - 1; }
};

// Largest number of blocks that contribute to one (tile, matrix) of a line of
// n_tm (tile, matrix) pairs of nsb units each, split over Wc compute waves.
int plan_cmax(long n_tm, int nsb, int Wc) {
  const UnitSplit sp(n_tm * nsb, Wc);
  long cmax = 1;
  for (long tm = 0; tm < n_tm; ++tm)
    cmax = std::max(cmax, sp.wave_of(tm * nsb + nsb - 1) / kCompute - sp.wave_of(tm * nsb) / kCompute + 1);
  return (int)cmax;
}

StepLayout layout(const mk_stack* st, int T) {
  StepLayout y;
  const mk_stack_desc& d = st->d;
  int dev = 0, cu = 256;
  hipGetDevice(&dev);
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) == hipSuccess) cu = p.multiProcessorCount;
  int per_cu = 0;
  StepKernel k = step_kernel(T);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k, kBlock, 0) != hipSuccess) per_cu = 0;
  y.grid = per_cu >= 1 ? cu : 0;  // one block (7 compute waves + 1 service wave) per CU
  y.Wc = y.grid * kCompute;
  const int ntiles[4] = {d.proj / 64, d.hidden / 64, d.ffn / 64, d.hidden / 64};
  const int nms[4] = {1, 1, 2, 1};
  const int nsbs[4] = {d.hidden / 256, d.proj / 256, d.hidden / 256, d.ffn / 256};
  for (int i = 0; i < 4; ++i) y.cmax[i] = y.Wc ? plan_cmax((long)ntiles[i] * nms[i], nsbs[i], y.Wc) : 1;
  // (each count must fit a byte of the packed kernel argument)
  // activation records: kActBytes per superblock of each input (x, u, x2, h)
  const int halves = T > 16 ? 2 : 1;  // 16-row record halves, lm streams
  auto rec = [halves](int K) { return (size_t)(K / 256) * kActBytes * halves; };
  y.act_off[K_X] = 0;
  y.act_off[K_U] = rec(d.hidden);
  y.act_off[K_X2] = y.act_off[K_U] + rec(d.proj);
  y.act_off[K_H] = y.act_off[K_X2] + rec(d.hidden);
  y.act_layer = y.act_off[K_H] + rec(d.ffn);
  size_t o = 0;
  y.off_ctrl = o;
  o += 256;  // barrier counter
  y.off_lmticket = o;
  o += 256;
  y.off_rdy = o;
  o += a256((size_t)(4 * d.n_layers + 1) * kRdySlots * kRdyStride * 4);
  y.off_open = o;
  o += a256((size_t)std::max(y.grid, 1) * kRdyStride * 4);
  y.off_tickets = o;
  o += a256((size_t)d.n_layers * 4 * kTicketTiles * kTicketStride * 4);
  y.n_ctrl = o - y.off_ctrl;
  y.off_out = o;
  o += a256(kOutWords * 4);
  y.off_stamps = o;
  o += a256(sizeof(uint64_t) * kMaxStamps);
  y.off_tag = o;
  o += 256;
  y.off_table = o;
  o += a256(sizeof(LayerW) * d.n_layers);
  y.off_plans = o;
  o += a256(sizeof(BlockPlan) * std::max(y.grid, 1));
  y.off_act = o;
  o += y.act_layer * d.n_layers;
  y.off_ss = o;
  o += a256((size_t)(2 * d.n_layers + 1) * (d.hidden / 64) * (T > 16 ? 32 : 16) * 4);
  y.off_part = o;
  size_t part = 0;
  const int tp = (T + 3) & ~3;
  for (int i = 0; i < 4; ++i) part = std::max(part, (size_t)ntiles[i] * nms[i] * y.cmax[i] * tp * 64 * 4);
  y.part_half = a256(part) / 4;  // floats; two buffers, by phase parity
  o += 2 * a256(part);
  y.off_frag = o;
  y.frag_half = a256((size_t)(d.hidden / 64) * 64 * 32 * 2) / 2;
  o += halves * y.frag_half * 2;
  y.off_lmv = o;
  o += a256((size_t)y.grid * 16 * 4 * halves);
  y.off_lmi = o;
  o += a256((size_t)y.grid * 16 * 4 * halves);
  y.total = o;
  return y;
}

int sfail(int status, const char* msg) { return set_error(status, "%s", msg); }

// The split of every phase kind's line of units over the grid's compute
// waves (UnitSplit), written per block:
// each compute wave's range, the (tile, matrix) pairs the block contributes
// to with the waves and the rank of its contribution, and the tiles it owns
// (tile tau by block tau * grid / n_tiles) with their contributor counts.
// Returns false when a block would exceed the plan's fixed capacities.
bool make_plans(const mk_stack_desc& d, int grid, std::vector<BlockPlan>& out) {
  const long Wc = (long)grid * kCompute;
  const int ntiles[4] = {d.proj / 64, d.hidden / 64, d.ffn / 64, d.hidden / 64};
  const int nms[4] = {1, 1, 2, 1};
  const int nsbs[4] = {d.hidden / 256, d.proj / 256, d.hidden / 256, d.ffn / 256};
  out.assign(grid, BlockPlan());
  memset(out.data(), 0, sizeof(BlockPlan) * out.size());
  for (int k = 0; k < 4; ++k) {
    const long nsb = nsbs[k], S = (long)ntiles[k] * nms[k] * nsb;
    const UnitSplit sp(S, Wc);
    auto lo = [&](long w) { return sp.lo[w]; };
    auto wave_of = [&](long p) { return sp.wave_of(p); };
    auto first_block = [&](long tm) { return wave_of(tm * nsb) / kCompute; };
    auto n_blocks = [&](long tm) { return wave_of(tm * nsb + nsb - 1) / kCompute - first_block(tm) + 1; };
    for (int b = 0; b < grid; ++b) {
      BlockPlan& p = out[b];
      for (int c = 0; c < kCompute; ++c) {
        const long w = (long)b * kCompute + c, u = lo(w), u1 = lo(w + 1);
        p.wu[k][c][0] = (int)u;
        p.wu[k][c][1] = (int)u1;
        p.wu[k][c][2] = u < u1 ? (int)(u / nsb) : 0;
        p.wu[k][c][3] = u < u1 ? (int)(u % nsb) : 0;
      }
      const long ub0 = lo((long)b * kCompute), ub1 = lo((long)(b + 1) * kCompute);
      int tm0 = 0, ntm = 0;
      if (ub0 < ub1) {
        tm0 = (int)(ub0 / nsb);
        ntm = (int)((ub1 - 1) / nsb) - tm0 + 1;
        if (ntm > kMaxTm) return false;
        for (int i = 0; i < ntm; ++i) {
          const long tm = tm0 + i;
          const long p0 = std::max(tm * nsb, ub0), p1 = std::min((tm + 1) * nsb, ub1);
          const long clo = wave_of(p0) - (long)b * kCompute, chi = wave_of(p1 - 1) - (long)b * kCompute;
          const long rank = b - first_block(tm);
          if (clo < 0 || chi >= kCompute || rank < 0 || rank > 255) return false;
          p.tmc[k][i][0] = (uint8_t)clo;
          p.tmc[k][i][1] = (uint8_t)chi;
          p.tmc[k][i][2] = (uint8_t)rank;
        }
      }
      const int own0 = (int)((long)ntiles[k] * b / grid), own1 = (int)((long)ntiles[k] * (b + 1) / grid);
      if (own1 - own0 > kMaxOwn) return false;
      for (int o = 0; o < own1 - own0; ++o) {
        const long tau = own0 + o;
        const long n0 = n_blocks(tau * nms[k]), n1 = nms[k] == 2 ? n_blocks(tau * nms[k] + 1) : 0;
        if (n0 > 255 || n1 > 255) return false;
        p.oc[k][o][0] = (uint8_t)n0;
        p.oc[k][o][1] = (uint8_t)n1;
      }
      p.kp[k][0] = tm0;
      p.kp[k][1] = ntm;
      p.kp[k][2] = own0;
      p.kp[k][3] = own1 - own0;
    }
  }
  return true;
}

// The attention items of a step: positions per split (a multiple of 64),
// splits per (agent, KV head) and the first item of each agent in a layer.
// The items of all attention layers are dealt to the grid's GDN waves; the
// split is chosen so that each wave gets about 16 items and no item is
// shorter than 4 tiles.
struct AttnStepPlan {
  int chunk, per;
  int nsplit[kMaxAgents], item0[kMaxAgents + 1];
  size_t part_bytes, ticket_bytes;
};

int attn_check(const mk_step_attn* at, int T, const std::vector<int>& gs, int G, AttnStepPlan& p) {
  if (!at || at->n_layers < 1) return sfail(MK_ERR_ARG, "attention: no layers");
  if (at->Hq < 1 || at->Hkv < 1 || at->Hq % at->Hkv) return sfail(MK_ERR_SHAPE, "attention: Hq must be a multiple of Hkv");
  if (at->cap <= 0 || at->cap % 64) return sfail(MK_ERR_SHAPE, "attention: cap must be a positive multiple of 64");
  if (at->cap > MK_ATTN_CAP_MAX) return sfail(MK_ERR_RANGE, "attention: cap above MK_ATTN_CAP_MAX");
  if (G > kMaxAgents) return sfail(MK_ERR_RANGE, "attention: at most 16 agents");
  if (!at->h_ctx || !at->q || !at->o) return sfail(MK_ERR_ARG, "attention: null pointer");
  const bool f16 = at->k_cache || at->v_cache;
  const bool q8 = at->k_codes || at->k_scales || at->v_codes || at->v_scales;
  if (f16 == q8) return sfail(MK_ERR_ARG, "attention: give either the fp16 or the q8_0 cache");
  if (f16 && !(at->k_cache && at->v_cache)) return sfail(MK_ERR_ARG, "attention: fp16 cache pointer missing");
  if (q8 && !(at->k_codes && at->k_scales && at->v_codes && at->v_scales))
    return sfail(MK_ERR_ARG, "attention: q8_0 cache pointer missing");
  const void* ptrs[9] = {at->q, at->gate, at->k_cache, at->v_cache, at->o, at->k_codes, at->k_scales, at->v_codes,
                         at->v_scales};
  for (const void* q : ptrs)
    if ((uintptr_t)q % 16) return sfail(MK_ERR_ALIGN, "attention: a buffer is not 16-B aligned");
  const int gqa = at->Hq / at->Hkv;
  long W = 0;
  for (int g = 0; g < G; ++g) {
    const int ng = gs[g + 1] - gs[g];
    if (ng * gqa > 16) return sfail(MK_ERR_SHAPE, "attention: an agent's rows x Hq/Hkv exceed 16 query columns");
    if (at->h_ctx[g] < 0 || (long)at->h_ctx[g] + ng > at->cap)
      return sfail(MK_ERR_RANGE, "attention: cached positions + new rows exceed cap");
    W += ((long)at->h_ctx[g] + ng) * at->Hkv;
  }
  const long target = 16L * 256;  // items over the step
  long chunk = ((long)at->n_layers * W + target - 1) / target;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk < 4 * 64) chunk = 4 * 64;
  p.chunk = (int)chunk;
  p.item0[0] = 0;
  for (int g = 0; g < G; ++g) {
    const long L = (long)at->h_ctx[g] + (gs[g + 1] - gs[g]);
    p.nsplit[g] = (int)((L + chunk - 1) / chunk);
    p.item0[g + 1] = p.item0[g] + p.nsplit[g] * at->Hkv;
  }
  p.per = p.item0[G];
  p.part_bytes = a256((size_t)at->n_layers * p.per * (16 * 128 + 32) * 4);
  p.ticket_bytes = a256((size_t)at->n_layers * G * at->Hkv * 64);
  (void)T;
  return MK_OK;
}

int valid_q(const mk_q4k& w, int n_out, int n_in) {
  return w.blocks && w.n_out == n_out && w.n_in == n_in && ((uintptr_t)w.blocks % 256) == 0;
}

}  // namespace

extern "C" {

int mk_stack_create(const mk_stack_desc* desc, mk_stack** out) {
  if (!desc || !out) return sfail(MK_ERR_ARG, "stack: null argument");
  *out = nullptr;
  const mk_stack_desc& d = *desc;
  if (d.n_layers < 1 || d.n_layers > kMaxLayers) return sfail(MK_ERR_RANGE, "stack: n_layers outside 1..128");
  if (d.hidden <= 0 || d.proj <= 0 || d.ffn <= 0 || d.hidden % 256 || d.proj % 256 || d.ffn % 256)
    return sfail(MK_ERR_SHAPE, "stack: hidden, proj, ffn must be positive multiples of 256");
  if (d.hidden > 64 * kTicketTiles || d.proj > 64 * kTicketTiles || d.ffn > 64 * kTicketTiles)
    return sfail(MK_ERR_SHAPE, "stack: widths above 32768");
  if (d.vocab <= 0 || !d.lm_head || ((uintptr_t)d.lm_head % 16))
    return sfail(MK_ERR_ARG, "stack: lm_head missing or misaligned");
  if (!d.p_in || !d.p_out || !d.gate || !d.up || !d.down) return sfail(MK_ERR_ARG, "stack: null weight array");
  mk_stack* st = new mk_stack();
  st->d = d;
  st->layers.resize(d.n_layers);
  for (int l = 0; l < d.n_layers; ++l) {
    if (!valid_q(d.p_in[l], d.proj, d.hidden) || !valid_q(d.p_out[l], d.hidden, d.proj) ||
        !valid_q(d.gate[l], d.ffn, d.hidden) || !valid_q(d.up[l], d.ffn, d.hidden) ||
        !valid_q(d.down[l], d.hidden, d.ffn)) {
      delete st;
      return sfail(MK_ERR_SHAPE, "stack: a layer weight has the wrong shape, is null or misaligned");
    }
    const mk_q4k* ws[5] = {&d.p_in[l], &d.p_out[l], &d.gate[l], &d.up[l], &d.down[l]};
    for (int i = 0; i < 5; ++i) st->layers[l].w[i] = (const uint8_t*)ws[i]->blocks;
  }
  memset(st->gdn_idx, -1, sizeof(st->gdn_idx));
  st->gdn_flag.assign(d.n_layers, 0);
  if (d.h_gdn_layer)
    for (int l = 0; l < d.n_layers; ++l)
      if (d.h_gdn_layer[l]) {
        st->gdn_flag[l] = 1;
        st->gdn_idx[l] = (int8_t)st->n_gdn_layers++;
      }
  if (st->n_gdn_layers) {
    if (d.n_agents < 1 || d.n_agents > kMaxAgents || !d.dn) {
      delete st;
      return sfail(MK_ERR_ARG, "stack: GDN layers need 1..16 agent states");
    }
    for (int g = 0; g < d.n_agents; ++g) {
      const mk_deltanet& s = d.dn[g];
      if (!s.S || !s.ring || !s.n_acc || s.dk != 128 || s.dv != 128 ||
          s.nh != st->n_gdn_layers * kGdnHeadsPerLayer || s.T_max < 2 || s.T_max > MK_T_MAX) {
        delete st;
        return sfail(MK_ERR_SHAPE, "stack: agent state must have dk = dv = 128, nh = gdn layers * 32 and 2 <= T_max <= 16");
      }
      st->dn.push_back(s);
    }
  }
  st->tag = g_next_tag.fetch_add(1);
  if (hipEventCreate(&st->ev[0]) != hipSuccess || hipEventCreate(&st->ev[1]) != hipSuccess) {
    st->ev[0] = st->ev[1] = nullptr;
  }
  *out = st;
  return MK_OK;
}

void mk_stack_destroy(mk_stack* st) {
  if (!st) return;
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    for (auto it = g_ws_tables.begin(); it != g_ws_tables.end();)
      it = it->second == st->tag ? g_ws_tables.erase(it) : std::next(it);
  }
  for (int i = 0; i < 2; ++i)
    if (st->ev[i]) hipEventDestroy(st->ev[i]);
  if (st->hout) hipHostFree(st->hout);
  delete st;
}

float mk_decode_step_last_ms(const mk_stack* st) { return st ? st->last_ms : -1.0f; }

size_t mk_decode_step_workspace(const mk_stack* st, int32_t T) {
  if (!st || T < 1 || T > kStepTMax) return 0;
  return layout(st, T).total;
}

int mk_decode_step(mk_stack* st, float* x, int32_t T, const int32_t* h_group_start, int32_t G,
                   const int32_t* drafts, const float* gdn_q, const float* gdn_k, const float* gdn_v,
                   const float* gdn_g, const float* gdn_beta, float* gdn_o, int32_t* h_tokens, int32_t* h_n_acc,
                   int32_t* d_argmax, float* trace, void* ws, size_t ws_bytes, void* stream) {
  return mk_decode_step_attn(st, x, T, h_group_start, G, drafts, gdn_q, gdn_k, gdn_v, gdn_g, gdn_beta, gdn_o,
                             h_tokens, h_n_acc, d_argmax, trace, nullptr, ws, ws_bytes, stream);
}

size_t mk_decode_step_attn_workspace(const mk_stack* st, int32_t T, const int32_t* h_group_start, int32_t G,
                                     const mk_step_attn* attn) {
  if (!st || T < 1 || T > kStepTMax) return 0;
  const size_t base = layout(st, T).total;
  if (!attn) return base;
  std::vector<int> gs;
  if (!h_group_start) {
    if (G != 1) return 0;
    gs = {0, T};
  } else {
    if (G < 1 || G > MK_LM_MAX_G) return 0;
    gs.assign(h_group_start, h_group_start + G + 1);
  }
  AttnStepPlan ap;
  if (attn_check(attn, T, gs, G, ap) != MK_OK) return 0;
  return base + ap.part_bytes + ap.ticket_bytes;
}

int mk_decode_step_attn(mk_stack* st, float* x, int32_t T, const int32_t* h_group_start, int32_t G,
                        const int32_t* drafts, const float* gdn_q, const float* gdn_k, const float* gdn_v,
                        const float* gdn_g, const float* gdn_beta, float* gdn_o, int32_t* h_tokens, int32_t* h_n_acc,
                        int32_t* d_argmax, float* trace, const mk_step_attn* attn, void* ws, size_t ws_bytes,
                        void* stream) {
  if (!st) return sfail(MK_ERR_ARG, "decode: null stack");
  if (T < 1 || T > kStepTMax) return sfail(MK_ERR_RANGE, "decode: T outside 1..24");
  if (!x || ((uintptr_t)x % 16)) return sfail(MK_ERR_ALIGN, "decode: x null or misaligned");
  if (!h_tokens || !h_n_acc) return sfail(MK_ERR_ARG, "decode: null host output");
  std::vector<int> gs;
  if (!h_group_start) {
    if (G != 1) return sfail(MK_ERR_ARG, "decode: h_group_start null but G != 1");
    gs = {0, T};
  } else {
    if (G < 1 || G > MK_LM_MAX_G || G > T) return sfail(MK_ERR_RANGE, "decode: G outside 1..min(T, 16)");
    gs.assign(h_group_start, h_group_start + G + 1);
    if (gs[0] != 0 || gs[G] != T) return sfail(MK_ERR_RANGE, "decode: group starts must run from 0 to T");
    for (int g = 0; g < G; ++g)
      if (gs[g + 1] <= gs[g]) return sfail(MK_ERR_RANGE, "decode: empty group");
  }
  if (T > G && !drafts) return sfail(MK_ERR_ARG, "decode: drafts null");
  const bool gdn = st->n_gdn_layers > 0;
  if (gdn) {
    if (G != (int)st->dn.size()) return sfail(MK_ERR_ARG, "decode: G must equal the number of agent states");
    if (!gdn_q || !gdn_k || !gdn_v || !gdn_g || !gdn_beta || !gdn_o)
      return sfail(MK_ERR_ARG, "decode: GDN inputs/outputs missing");
    for (int g = 0; g < G; ++g)
      if (gs[g + 1] - gs[g] > st->dn[g].T_max) return sfail(MK_ERR_RANGE, "decode: group longer than its T_max");
  }
  AttnStepPlan ap = {};
  if (attn) {
    const int r = attn_check(attn, T, gs, G, ap);
    if (r != MK_OK) return r;
  }
  const StepLayout y = layout(st, T);
  if (y.grid < 1) return sfail(MK_ERR_COOP, "decode: the step kernel does not fit on a compute unit");
  const size_t need = y.total + (attn ? ap.part_bytes + ap.ticket_bytes : 0);
  if (!ws || ws_bytes < need) return set_error(MK_ERR_WORKSPACE, "decode: workspace %zu < %zu bytes", ws_bytes, need);
  if ((uintptr_t)ws % 256) return sfail(MK_ERR_ALIGN, "decode: workspace not 256-B aligned");
  hipStream_t s = (hipStream_t)stream;
  uint8_t* w8 = (uint8_t*)ws;
  bool fresh_plans = false;
  if (st->plans_grid != y.grid) {
    if (!make_plans(st->d, y.grid, st->plans)) return sfail(MK_ERR_SHAPE, "decode: shapes too small for the grid's work plan");
    st->plans_grid = y.grid;
    fresh_plans = true;
  }
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    auto it = g_ws_tables.find(ws);
    if (fresh_plans || it == g_ws_tables.end() || it->second != st->tag) {
      if (hipMemcpyAsync(w8 + y.off_table, st->layers.data(), sizeof(LayerW) * st->layers.size(),
                         hipMemcpyHostToDevice, s) != hipSuccess ||
          hipMemcpyAsync(w8 + y.off_plans, st->plans.data(), sizeof(BlockPlan) * st->plans.size(),
                         hipMemcpyHostToDevice, s) != hipSuccess ||
          hipMemcpyAsync(w8 + y.off_tag, &st->tag, sizeof(uint64_t), hipMemcpyHostToDevice, s) != hipSuccess) {
        g_ws_tables.erase(ws);
        return sfail(MK_ERR_LAUNCH, "decode: weight table upload failed");
      }
      g_ws_tables[ws] = st->tag;
    }
  }
  // the output block follows the control words: one reset for both
  if (y.off_out != y.off_ctrl + y.n_ctrl) return sfail(MK_ERR_LAUNCH, "decode: workspace layout");
  if (hipMemsetAsync(w8 + y.off_ctrl, 0, y.n_ctrl + kOutWords * 4, s) != hipSuccess ||
      (attn && hipMemsetAsync(w8 + y.total + ap.part_bytes, 0, ap.ticket_bytes, s) != hipSuccess))
    return sfail(MK_ERR_LAUNCH, "decode: control reset failed");
  StepArgs a;
  memset(&a, 0, sizeof(a));
  const mk_stack_desc& d = st->d;
  a.L = d.n_layers;
  a.H = d.hidden;
  a.P = d.proj;
  a.F = d.ffn;
  a.V = d.vocab;
  a.T = T;
  a.G = G;
  for (int i = 0; i <= MK_LM_MAX_G; ++i) a.gs[i] = i <= G ? gs[i] : T;
  a.Wc = y.Wc;
  a.cmax4 = 0;
  for (int i = 0; i < 4; ++i) a.cmax4 |= y.cmax[i] << (8 * i);
  a.layers = (const LayerW*)(w8 + y.off_table);
  a.plans = (const BlockPlan*)(w8 + y.off_plans);
  a.lm = d.lm_head;
  for (int l = 0; l < d.n_layers; ++l)
    if (st->gdn_flag[l]) a.gdn_mask[l >> 6] |= 1ull << (l & 63);
  memcpy(a.gdn_idx, st->gdn_idx, sizeof(a.gdn_idx));
  a.n_agents = gdn ? G : 0;
  if (gdn) {
    a.T_max = st->dn[0].T_max;
    a.nh = st->dn[0].nh;
    for (int g = 0; g < G; ++g) {
      if (st->dn[g].T_max != a.T_max) return sfail(MK_ERR_ARG, "decode: agent states need one T_max");
      a.S[g] = st->dn[g].S;
      a.ring[g] = st->dn[g].ring;
      a.nacc[g] = st->dn[g].n_acc;
    }
  }
  a.gq = gdn_q;
  a.gk = gdn_k;
  a.gv = gdn_v;
  a.gg = gdn_g;
  a.gb = gdn_beta;
  a.go = gdn_o;
  a.x = x;
  a.trace = trace;
  a.drafts = drafts;
  a.bar = (unsigned*)(w8 + y.off_ctrl);
  a.lm_ticket = (unsigned*)(w8 + y.off_lmticket);
  a.tickets = (unsigned*)(w8 + y.off_tickets);
  a.rdy = (unsigned*)(w8 + y.off_rdy);
  a.open = (unsigned*)(w8 + y.off_open);
  a.part_half = y.part_half;
  a.out = (int32_t*)(w8 + y.off_out);
  a.err = a.out;
  a.stamps = (uint64_t*)(w8 + y.off_stamps);
  a.act = w8 + y.off_act;
  a.act_layer = y.act_layer;
  for (int i = 0; i < 4; ++i) {
    a.act_off[i] = y.act_off[i];
  }
  a.ss = (float*)(w8 + y.off_ss);
  a.part = (float*)(w8 + y.off_part);
  a.frag = (_Float16*)(w8 + y.off_frag);
  a.frag_half = y.frag_half;
  a.lm_val = (float*)(w8 + y.off_lmv);
  a.lm_idx = (int*)(w8 + y.off_lmi);
  a.ws_tag = (const uint64_t*)(w8 + y.off_tag);
  a.tag = st->tag;
  // |RMSNorm(x)_i| <= sqrt(hidden) for every row, so 2^k with
  // sqrt(hidden) * 2^k <= 2^14 keeps every lm_head input far inside fp16's
  // range; the scaling is exact and leaves the argmax unchanged.
  a.lm_pre = ldexpf(1.0f, (int)floor(log2(16384.0 / sqrt((double)d.hidden))));
  if (attn) {
    a.n_attn = attn->n_layers;
    a.attn_Hq = attn->Hq;
    a.attn_Hkv = attn->Hkv;
    a.attn_gqa = attn->Hq / attn->Hkv;
    a.attn_cap = attn->cap;
    a.attn_chunk = ap.chunk;
    for (int g = 0; g < G; ++g) {
      a.attn_ctx[g] = attn->h_ctx[g];
      a.attn_nsplit[g] = ap.nsplit[g];
    }
    for (int g = 0; g <= kMaxAgents; ++g) a.attn_item0[g] = g <= G ? ap.item0[g] : ap.item0[G];
    a.attn_qscale = (float)(1.4426950408889634 / sqrt(128.0));  // log2(e) / sqrt(d)
    a.attn_q = attn->q;
    a.attn_gate = attn->gate;
    a.attn_k = attn->k_cache;
    a.attn_v = attn->v_cache;
    a.attn_k8 = attn->k_codes;
    a.attn_ks = attn->k_scales;
    a.attn_v8 = attn->v_codes;
    a.attn_vs = attn->v_scales;
    a.attn_q8 = attn->k_codes != nullptr;
    a.attn_o = attn->o;
    a.attn_part = (float*)(w8 + y.total);
    a.attn_ticket = (unsigned*)(w8 + y.total + ap.part_bytes);
  }
  void* args[] = {&a};
  if (st->ev[0]) hipEventRecord(st->ev[0], s);
  hipError_t e = hipLaunchCooperativeKernel((const void*)step_kernel(T, attn != nullptr), dim3(y.grid),
                                            dim3(kBlock), args, 0, s);
  if (st->ev[1]) hipEventRecord(st->ev[1], s);
  if (e != hipSuccess)
    return set_error(e == hipErrorCooperativeLaunchTooLarge ? MK_ERR_COOP : MK_ERR_LAUNCH,
                     "decode: cooperative launch failed: %s", hipGetErrorString(e));
  if (d_argmax &&
      hipMemcpyAsync(d_argmax, w8 + y.off_out + kOutTop * 4, T * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return sfail(MK_ERR_LAUNCH, "decode: argmax copy failed");
  // read back into pinned memory (one DMA; a pageable copy is staged)
  if (!st->hout && hipHostMalloc((void**)&st->hout, kOutWords * 4, hipHostMallocDefault) != hipSuccess) st->hout = nullptr;
  int32_t hlocal[kOutWords];
  int32_t* hout = st->hout ? st->hout : hlocal;
  if (hipMemcpyAsync(hout, w8 + y.off_out, kOutWords * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return sfail(MK_ERR_LAUNCH, "decode: readback failed");
  st->last_ms = -1.0f;
  if (st->ev[0] && st->ev[1]) hipEventElapsedTime(&st->last_ms, st->ev[0], st->ev[1]);
  if (hout[0] & kErrTables) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    g_ws_tables.erase(ws);
    return sfail(MK_ERR_WORKSPACE,
                 "decode: the workspace no longer holds this stack's tables (another call wrote it); nothing ran, "
                 "the next call uploads them again");
  }
  if (hout[0] & kErrWatchdog) return sfail(MK_ERR_DEVICE, "decode: a bounded wait in the step ran out (watchdog)");
  if (hout[0] & kErrAccept)
    return sfail(MK_ERR_RANGE, "decode: an agent state's accept length was outside 0..T_max-1 (nothing was replayed)");
  if (hout[0]) return sfail(MK_ERR_DEVICE, "decode: device error word set");
  for (int g = 0; g < G; ++g) h_n_acc[g] = hout[kOutNacc + g];
  for (int t = 0; t < T; ++t) h_tokens[t] = hout[kOutTok + t];
  set_error(MK_OK, "");
  return MK_OK;
}

int mk_decode_step_stamps(const mk_stack* st, int32_t T, const void* ws, uint64_t* h_stamps, int32_t n,
                          int64_t* h_clock_hz) {
  if (!st || !ws || !h_stamps || n < 1) return sfail(MK_ERR_ARG, "stamps: null argument");
  const StepLayout y = layout(st, T);
  const int m = n < kMaxStamps ? n : kMaxStamps;
  if (hipMemcpy(h_stamps, (const uint8_t*)ws + y.off_stamps, sizeof(uint64_t) * m, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return sfail(MK_ERR_LAUNCH, "stamps: copy failed");
  if (h_clock_hz) {
    int dev = 0, khz = 0;
    hipGetDevice(&dev);
    hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    *h_clock_hz = (int64_t)khz * 1000;
  }
  return m;
}

}  // extern "C"
