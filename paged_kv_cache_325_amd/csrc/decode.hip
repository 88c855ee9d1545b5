// Paged GQA decode with split-K (flash-decoding) for gfx950.
//
// Operation (nano-vllm source study, section 2: decode attention over the
// paged KV cache with per-sequence context lengths and block tables; vLLM
// essay, section 3.2: translate logical positions to (block, row), gather,
// compute): for sequence b and query head h, with g = h / (Hq/Hkv) and
// n = context_lens[b],
//     out[b][h] = sum_{j<n} softmax_j(scale * q[b][h] . K_j) V_j,
//     K_j = k_cache[block_tables[b][j / 256]][g][j % 256].
//
// Work decomposition.  One workgroup is ONE wavefront and owns (split s,
// sequence b, kv head g, chunk of heads_per_wg query heads of g's group).  It
// walks the keys s*S .. min(n,(s+1)*S)-1 in chunks of 64 (32 for fp32)
// tokens.  A chunk never crosses a 256-token block, and in the
// [block][kv head][row][dim] layout its K rows (and V rows) for kv head g are
// one contiguous 16 KiB run, read once per chunk for all heads of the group.
//
// Per chunk:
//   1. K and V rows are loaded with fully coalesced 16-byte loads (each wave
//      load instruction reads 1 KiB contiguous).  K goes to LDS with rows
//      padded by 16 bytes.
//   2. QK: lane t owns token t and reads its whole K row back from LDS
//      (the padding makes 16 consecutive rows hit 16 different bank groups);
//      q comes from LDS as a broadcast.  bf16 uses v_dot2_f32_bf16, so no
//      conversion and no cross-lane reduction is needed for the scores.
//   3. Online softmax in base 2 (x = scale*log2(e)*score): the chunk max is a
//      wave reduction, p = 2^(x - m) is computed once per (token, head).
//   4. PV: V stays in the registers it was loaded into -- lane l holds 8 (4)
//      consecutive dims of token 4i + l/16 (2i + l/32) -- and takes p from
//      LDS; the token groups are summed once at the end of the split.
// Rows past the context inside the last block are read (they are inside the
// allocation) but their score is replaced by -inf and their V by 0, so NaN
// poison there cannot leak.
//
// Each split writes unnormalised (acc, m, l) to the workspace; a second,
// small kernel merges them in split order (deterministic).  A sequence with
// a single split writes its output directly.  The kernel boundary is what
// makes the partials of every XCD visible to the merge: merging inside the
// split kernel would need an agent-scope release/acquire (a full L2
// write-back and invalidate) in every split, which costs far more than the
// second launch.  HBM-bound: the algorithmic traffic is
// the context's K and V bytes plus q and out.
#include <math.h>

#include <algorithm>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

// Workgroups the automatic split plan aims for.  The plan is a function of
// the arguments only -- not of the device -- so that
// pkv_paged_decode_workspace_bytes can size the workspace on the host
// without a device query and results do not change between parts; the
// targets are tuned for the 256 CUs of MI355X.  Large batches: 8192, 32 per
// CU, enough for balance.  Small batches: 1024, so each workgroup
// streams several chunks and its loads overlap its compute -- used while
// that leaves at most kSmallPlanChunks 64-token chunks per workgroup.
// Measured on the 28-layer fused decode step (graph-replayed, 16 / 8
// query / kv heads, contexts of 512-4096): 1024 workgroups beat 8192 by
// 8-15 % at batches 4-16 and ~3 % at 32; 8192 stays best at 64.
constexpr int kTargetWaves = 256 * 32;
// Compacted units (unit_of) cost each split workgroup ~1 us of latency
// before its first load; they pay where the grid holds many empty units
// (max_context_len spans at least kMinCompactSplits splits, so sequences
// shorter than it leave most of theirs empty) and each unit carries
// enough keys to hide that latency (kMinCompactSplit).  Measured with
// interleaved A/B runs (bitwise-equal outputs): the 16-sequence
// lognormal-length workload (64 splits of 512 keys) 125.7 -> 117.3 us; the
// 64- and 256-sequence workloads (16 splits of 256 keys, 4 of 2048) within
// 0.5 %; 28-layer graph-replayed steps at batch 16 (8 splits of 512 keys)
// 4 % slower, at batch 2-8 (64-256-key splits) unchanged -- hence the
// bounds.  Putting the ragged last splits after all full ones took the
// lognormal workload's decode from 124.1 to 119.5 us (bitwise equal); with
// looser bounds (4 splits of 256 keys) the 64- and 256-sequence workloads
// and batches 8-16 were 1-3 % slower.
constexpr int kMaxCompactBatch = 256;
constexpr int kMinCompactSplits = 16;
constexpr int kMaxCompactSplits = 1024;
constexpr int kMinCompactSplit = 512;
constexpr int kSmallTargetWaves = 1024;
constexpr int kSmallPlanChunks = 16;

template <int kElemBytes>
struct DecodeShape {
  static constexpr int kVec = 16 / kElemBytes;            // elements per 16-byte chunk
  static constexpr int kChunksPerRow = kHeadDim / kVec;   // 16 (bf16) or 32 (fp32)
  static constexpr int kRowBytes = kHeadDim * kElemBytes;  // 256 or 512
  static constexpr int kRowsPerLoad = 64 / kChunksPerRow;  // rows per wave load: 4 or 2
  static constexpr int kTokens = (kElemBytes == 2) ? 64 : 32;  // tokens per chunk
  static constexpr int kLoads = kTokens / kRowsPerLoad;        // 16 for both
};

struct DecodeArgs {
  const uint8_t* q;
  int64_t q_stride_bytes;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  int32_t batch, num_q_heads, num_kv_heads, group, head_chunks;
  FastDiv bdiv;       // block size (bdiv.d) and division by it
  int32_t bshift;     // log2(block size) when a chunk spans several blocks
  float scale_log2;
  int32_t split_tokens, nsplit;
  uint8_t* out;
  float* ws_acc;
  float* ws_ml;
  // Fused store (decode step): this step's K/V row of every sequence, stored
  // at slot_mapping[b] by the kernel itself; k_new == nullptr: no store.
  const uint8_t* k_new;
  const uint8_t* v_new;
  int64_t k_new_stride_bytes, v_new_stride_bytes;
  const int32_t* slot_mapping;
  uint8_t* k_cache_w;
  uint8_t* v_cache_w;
  // Shared-prefix plan (device words, layout in pkv_internal.h): the first
  // prefix_wgs = prefix_items * num_kv_heads workgroups attend the shared
  // splits; split workgroups skip the splits their sequence's subgroup
  // covers.  Used only by the kPrefix instantiations.
  const int32_t* prefix_plan;
  int32_t prefix_items, prefix_wgs;
  // Compacted units (see unit_of): split workgroups enumerate only the
  // (sequence, split) units that have work, in split-major order.
  int32_t compact;
  FastDiv sdiv;  // division by split_tokens
};

struct TrueTag { static constexpr bool value = true; };
struct FalseTag { static constexpr bool value = false; };

template <int kElemBytes>
__device__ __forceinline__ void unpack(const u32x4& w, float* f) {
  if constexpr (kElemBytes == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
}

// ---- shared splits of a subgroup (bf16, MFMA) ------------------------------
// A split that the sequences of a subgroup hold in the same physical blocks
// (equal leading block-table entries: hash-based prefix caching gives
// sequences with a common prompt prefix the same blocks) is attended once for
// all of them.  The members' query heads of kv head g are the columns of one
// v_mfma_f32_16x16x32_bf16 tile (at most 16: 16 / G members), the split's
// keys its rows.  Per 32-key chunk: the K and V rows arrive in registers
// (coalesced 1 KiB nontemporal loads, two chunks in flight), are staged in
// LDS, and
//   S^T (32 keys x 16 columns) = K Q^T      A: K rows from LDS, B: q
//   online softmax per column, base 2
//   O^T (128 dims x 16 columns) += V^T P^T  A: V^T by LDS transpose reads,
//                                           B: P^T straight from S^T
// MFMA layouts (16x16x32): lane l holds A[l%16][8(l/16)..+7],
// B[8(l/16)..+7][l%16] and D[4(l/16)..+3][l%16].  The keys of a chunk are
// ordered for the PV contraction as k = 8j + i -> key 4j + i (i < 4) and
// 16 + 4j + i - 4 (i >= 4), which is where S^T left them in lane 16j + n.
// Each member's (acc, m, l) is written to its own workspace slot of that
// split, so the merge treats it as any other split.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

// A staged chunk: 32 key rows x 16 chunks of 16 bytes, for K and for V, with
// chunk c of row r at position
//   K: c ^ (r & 15)  -- the 16 rows of one A-operand read hit 16 distinct
//                       16-byte bank groups;
//   V: c ^ 2(r & 7)  -- the 8 rows of one half-wave transpose read hit 8
//                       distinct 32-byte bank groups.
__device__ __forceinline__ int pk_pos(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int pv_pos(int r, int c) { return c ^ ((r & 7) << 1); }

// kSmall: blocks of 16 or 32 tokens (each 1 KiB load of 4 rows gets its own
// lookup); otherwise a 32-key chunk lies in one block.
template <bool kSmall>
__device__ __forceinline__ void prefix_split(const DecodeArgs& a, int id, u32x4* lds) {
  const int lane = threadIdx.x;
  const int g = id % a.num_kv_heads;
  const int item = id / a.num_kv_heads;
  const int32_t* plan = a.prefix_plan;
  // a plan built for another split length, batch or GQA group is ignored
  // (the split workgroups make the same test and then skip nothing)
  if (plan[0] != a.split_tokens || plan[1] != a.prefix_items || plan[2] != a.batch ||
      plan[3] != a.group)
    return;
  const int nsub = plan[4];
  const int32_t* groups = plan + kPlanHeader + a.batch;
  const int32_t* it = groups + (int64_t)kPlanGroupWords * nsub + 2 * item;
  const int sg = it[0], s = it[1];
  if (sg < 0 || sg >= nsub || s < 0 || s >= a.nsplit) return;
  const int32_t* rec = groups + (int64_t)kPlanGroupWords * sg;
  const int cnt = rec[0];
  const int G = a.group;
  if (cnt < 1 || cnt * G > kPlanMembers) return;

  const int n = lane & 15;  // column: member n / G, query head g*G + n % G
  const int j = lane >> 4;
  const bool col_ok = n < cnt * G;
  const int mi = col_ok ? n / G : 0;
  const int b_col = rec[1 + mi];
  const int h_col = g * G + (col_ok ? n - mi * G : 0);
  const int S = a.split_tokens;
  const int k_lo = s * S, k_hi = k_lo + S;

  // The plan must match the tables: every member holds the split before its
  // last position, in the same blocks.  A plan that does not (built for
  // other tables) gives NaN for the members' outputs instead of wrong rows.
  bool bad;
  {
    const int bi = lane < cnt ? rec[1 + lane] : 0;
    const bool id_ok = bi >= 0 && bi < a.batch;
    const int ni = (lane < cnt && id_ok) ? a.context_lens[bi] : 0x7fffffff;
    bad = __builtin_amdgcn_ballot_w64(lane < cnt && (!id_ok || ni <= k_hi)) != 0;
  }
  const uint32_t bs = a.bdiv.d;
  const int blk_lo = (int)a.bdiv.div((uint32_t)k_lo);
  const int nblk = (int)a.bdiv.div((uint32_t)(k_hi - 1)) - blk_lo + 1;
  bad |= nblk > 64;
  int tab = 0;
  if (!bad) {
    tab = lane < nblk ? a.block_tables[(int64_t)rec[1] * a.max_blocks + blk_lo + lane] : 0;
    for (int i = 1; i < cnt; ++i) {
      const int ti = lane < nblk ? a.block_tables[(int64_t)rec[1 + i] * a.max_blocks + blk_lo + lane] : 0;
      bad |= __builtin_amdgcn_ballot_w64(ti != tab) != 0;
    }
  }
  if (bad) {
    if (col_ok && j == 0 && b_col >= 0 && b_col < a.batch) {
      const int64_t slot = ((int64_t)b_col * a.num_q_heads + h_col) * a.nsplit + s;
      *reinterpret_cast<f32x2*>(a.ws_ml + slot * 2) = f32x2{NAN, NAN};
    }
    return;
  }

  // q^T columns: dims 32 ks + 8 j .. + 7 of the lane's column
  u32x4 qf[4];
  {
    const uint8_t* qp = a.q + (int64_t)b_col * a.q_stride_bytes + (int64_t)h_col * 256 + j * 16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = col_ok ? *reinterpret_cast<const u32x4*>(qp + ks * 64) : u32x4{0u, 0u, 0u, 0u};
  }

  // byte offset of key row kk (kv head g) in the cache
  auto row_base = [&](int kk) -> int64_t {
    const uint32_t q = a.bdiv.div((uint32_t)kk);
    const int64_t blk = __builtin_amdgcn_readlane(tab, (int)q - blk_lo);
    return ((blk * a.num_kv_heads + g) * bs + (kk - q * bs)) * 256;
  };
  auto load = [&](u32x4 (&kr)[8], u32x4 (&vr)[8], int t) {
    const int c0 = k_lo + 32 * t;
    if constexpr (kSmall) {
#pragma unroll
      for (int i = 0; i < 8; ++i) kr[i] = stream_load(a.k_cache + row_base(c0 + 4 * i) + lane * 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) vr[i] = stream_load(a.v_cache + row_base(c0 + 4 * i) + lane * 16);
    } else {
      const int64_t base = row_base(c0);
#pragma unroll
      for (int i = 0; i < 8; ++i) kr[i] = stream_load(a.k_cache + base + i * 1024 + lane * 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) vr[i] = stream_load(a.v_cache + base + i * 1024 + lane * 16);
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;
  const float c = a.scale_log2;
  u32x4* kl = lds;
  u32x4* vl = lds + 32 * 16;
  const int ta = lane & 3, tm = (lane >> 2) & 3;

  // One wave: its LDS accesses complete in order, so the previous chunk's
  // operand reads are done before the next chunk's rows land.  Lane l of
  // load i holds chunk l % 16 of row 4 i + l / 16.
  auto stage = [&](const u32x4 (&kr)[8], const u32x4 (&vr)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + j;
      kl[r * 16 + pk_pos(r, n)] = kr[i];
      vl[r * 16 + pv_pos(r, n)] = vr[i];
    }
  };
  auto compute = [&]() {
    f32x4 sc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * mt + n;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(kl[r * 16 + pk_pos(r, 4 * ks + j)]), as_bf16x8(qf[ks]), sc[mt], 0, 0, 0);
    }
    // online softmax of the lane's 8 keys; a column's 32 keys are spread
    // over lanes n, n + 16, n + 32, n + 48
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sc[e >> 2][e & 3] * c;
    float cm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
    const float mn = fmaxf(m_run, cm);
    const float alpha = fast_exp2(m_run - mn);
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(x[e] - mn);
    const u32x4 pf = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                           pack_bf16(p[6], p[7])};
    // the row sum of the bf16 probabilities the PV product consumes
    float ps = dot2_bf16(pf[0], kOnesBf16x2, 0.f);
    ps = dot2_bf16(pf[1], kOnesBf16x2, ps);
    ps = dot2_bf16(pf[2], kOnesBf16x2, ps);
    ps = dot2_bf16(pf[3], kOnesBf16x2, ps);
    l_lane = fmaf(l_lane, alpha, ps);
    m_run = mn;
    // the V^T operand reads are not hoisted above the softmax (registers)
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T.  ds_read_b64_tr_b16: in each 16-lane group, lane
    // 4a + e receives element e of the 8-byte chunks addressed by lanes a,
    // a + 4, a + 8, a + 12.  Lane 16 j + 4 tm + ta addresses key 4 j + tm
    // (then 16 + 4 j + tm) at dims 16 dt + 4 ta, so lane 16 j + d receives
    // dim 16 dt + d of keys 4 j .. 4 j + 3 (then 16 + 4 j ..).
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      o[dt] *= alpha;
      const int dim = 16 * dt + 4 * ta;
      const int r0 = 4 * j + tm, r1 = 16 + 4 * j + tm;
      const char* p0 = reinterpret_cast<const char*>(vl) + r0 * 256 + pv_pos(r0, dim >> 3) * 16 + (dim & 7) * 2;
      const char* p1 = reinterpret_cast<const char*>(vl) + r1 * 256 + pv_pos(r1, dim >> 3) * 16 + (dim & 7) * 2;
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0));
      const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}),
                                                      as_bf16x8(pf), o[dt], 0, 0, 0);
    }
  };

  // One chunk in registers: it is loaded while the previous one is computed
  // from LDS.
  u32x4 kr[8], vr[8];
  const int nch = S / 32;
  load(kr, vr, 0);
  for (int t = 0; t + 1 < nch; ++t) {
    stage(kr, vr);
    load(kr, vr, t + 1);
    compute();
  }
  stage(kr, vr);
  compute();

  float l_col = l_lane + __shfl_xor(l_lane, 16, 64);
  l_col += __shfl_xor(l_col, 32, 64);
  if (col_ok) {
    const int64_t slot = ((int64_t)b_col * a.num_q_heads + h_col) * a.nsplit + s;
    float* dst = a.ws_acc + slot * kHeadDim + 4 * j;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = o[dt];
    if (j == 0) *reinterpret_cast<f32x2*>(a.ws_ml + slot * 2) = f32x2{m_run, l_col};
  }
}

// kSmall: blocks shorter than a chunk (16 or 32 tokens, a power of two): each
// 1 KiB load of a chunk still lies in one block, but consecutive loads of a
// chunk may lie in different blocks, so each load gets its own block lookup.
// Otherwise a chunk lies in one block and one lookup serves all its loads.
// Compacted units.  The host knows only max_context_len, so the grid has
// nsplit units per sequence, and for skewed lengths most of them are empty:
// those workgroups, interleaved in the dispatch order, delayed the
// workgroups of the long sequences' last splits and so stretched the tail.
// Here unit u of the launch is the u-th (sequence, split) that has work:
// first every full split (S keys) in split-major order (the same split of
// different sequences runs together, as before), skipping the splits a
// shared-prefix subgroup computes, then each sequence's ragged last split
// (or the one unit of an empty context, which writes its zero row), the
// shorter units at the end of the dispatch; units past the last one exit.
// Every lane holds the counts of sequences lane + 64 k (batch <= 256, the
// host's condition); each row s of the walk costs a ballot per k.  Returns
// false for a unit past the end.
template <bool kPrefix>
__device__ __forceinline__ bool unit_of(const DecodeArgs& a, int u, int& b_out, int& s_out,
                                        int& n_out) {
  constexpr int kMaxK = kMaxCompactBatch / 64;
  const int lane = threadIdx.x;
  const int K = (a.batch + 63) >> 6;  // uniform, 1 .. kMaxK
  bool plan_ok = false;
  if constexpr (kPrefix) {
    const int32_t* plan = a.prefix_plan;
    plan_ok = plan[0] == a.split_tokens && plan[1] == a.prefix_items && plan[2] == a.batch &&
              plan[3] == a.group;
  }
  // full splits lo .. full-1 first (split-major), then each sequence's
  // ragged last split (or the zero row of an empty context) at s = full
  int nb[kMaxK], lo[kMaxK], full[kMaxK];
  bool rag[kMaxK];
  int mine = 0, nrag = 0;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    nb[k] = lo[k] = full[k] = 0;
    rag[k] = false;
    if (k < K) {
      const int bb = lane + 64 * k;
      const bool in = bb < a.batch;
      nb[k] = in ? a.context_lens[bb] : 0;
      full[k] = in ? (int)a.sdiv.div((uint32_t)nb[k]) : 0;
      rag[k] = in && (nb[k] == 0 || nb[k] != full[k] * a.split_tokens);
      if constexpr (kPrefix)
        lo[k] = (in && plan_ok) ? min(a.prefix_plan[kPlanHeader + bb], full[k]) : 0;
      mine += full[k] - lo[k];
      nrag += rag[k] ? 1 : 0;
    }
  }
  const int total1 = (int)wave_sum((float)mine);
  if (u >= total1) {
    int r = u - total1;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(rag[k]);
      const int c = __builtin_popcountll(m);
      if (r >= 0 && r < c) {
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        const uint64_t hit = __builtin_amdgcn_ballot_w64(((m >> lane) & 1) && rank == r);
        const int l = __builtin_ffsll((long long)hit) - 1;
        b_out = 64 * k + l;
        n_out = __builtin_amdgcn_readlane(nb[k], l);
        s_out = __builtin_amdgcn_readlane(full[k], l);
        return true;
      }
      r -= c;
    }
    return false;
  }
  // walk the rows (splits) to the one holding unit u
  int before = 0;
  for (int s = 0; s < a.nsplit; ++s) {
    uint64_t m[kMaxK];
    int row = 0;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      m[k] = 0;
      if (k < K) {
        m[k] = __builtin_amdgcn_ballot_w64(s >= lo[k] && s < full[k]);
        row += __builtin_popcountll(m[k]);
      }
    }
    if (u < before + row) {
      int r = u - before;
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        const int c = __builtin_popcountll(m[k]);
        if (r >= 0 && r < c) {
          const int rank = __builtin_amdgcn_mbcnt_hi(
              (uint32_t)(m[k] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[k], 0));
          const uint64_t hit = __builtin_amdgcn_ballot_w64(((m[k] >> lane) & 1) && rank == r);
          const int l = __builtin_ffsll((long long)hit) - 1;
          b_out = 64 * k + l;
          n_out = __builtin_amdgcn_readlane(nb[k], l);
        }
        r -= c;
      }
      s_out = s;
      return true;
    }
    before += row;
  }
  return false;
}

// kPrefix (bf16 only): the launch starts with the workgroups of a
// shared-prefix plan's items, and split workgroups skip the splits a
// subgroup covers.
template <int kElemBytes, int kHeads, bool kFused, bool kSmall, bool kPrefix>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  using S = DecodeShape<kElemBytes>;
  constexpr int kVec = S::kVec;
  constexpr int kCPR = S::kChunksPerRow;
  constexpr int kTok = S::kTokens;

  // K rows padded by one 16-byte column: row stride kCPR + 1 chunks
  __shared__ u32x4 k_lds[kTok * (kCPR + 1)];
  __shared__ u32x4 q_lds[kHeads * kCPR];
  __shared__ float p_lds[kTok * kHeads];

  const int lane = threadIdx.x;
  int id = blockIdx.x;
  if constexpr (kPrefix) {
    static_assert(kElemBytes == 2, "shared splits are bf16 only");
    if (id < a.prefix_wgs) {
      prefix_split<kSmall>(a, id, k_lds);
      return;
    }
    id -= a.prefix_wgs;
  }
  const int hc = id % a.head_chunks;
  id /= a.head_chunks;
  const int g = id % a.num_kv_heads;
  id /= a.num_kv_heads;
  int b, s, n;
  if (a.compact) {
    if (!unit_of<kPrefix>(a, id, b, s, n)) return;
  } else {
    b = id % a.batch;
    s = id / a.batch;
    n = a.context_lens[b];
  }
  const int start = s * a.split_tokens;
  const int h0 = g * a.group + hc * kHeads;
  // query heads of this chunk that exist: fewer than kHeads in the last
  // chunk when the group is not a multiple of kHeads (the rest compute on a
  // zero q and write nothing)
  const int nh = min(kHeads, a.group - hc * kHeads);

  // Fused store: the workgroup of head chunk 0 whose split holds the last
  // position writes the new row of kv head g to its slot, and every
  // workgroup whose split reads position n-1 takes that row from the input
  // instead of the cache (so no workgroup reads a cache row this launch
  // writes).  The decode-step invariant makes this exactly store-then-decode:
  // the slot is -1 or the slot of position n-1, in a block no other
  // sequence reads.
  // With 8 heads and blocks of 16 or 32 tokens the new row is not kept in
  // registers through the loop (those 8 VGPRs would push the kernel past 256,
  // one wave per SIMD instead of two): the last chunk reads it again from the
  // input, where it is cache-resident.
  constexpr bool kReloadNew = kHeads == 8 && kSmall;
  auto new_row = [&](const uint8_t* base, int64_t stride) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(base + b * stride + (int64_t)g * S::kRowBytes +
                                           (lane % kCPR) * 16);
  };
  int slot_new = -1;
  u32x4 knew = u32x4{0u, 0u, 0u, 0u}, vnew = u32x4{0u, 0u, 0u, 0u};
  if constexpr (kFused) {
    slot_new = a.slot_mapping[b];
    if (slot_new >= 0) {
      knew = new_row(a.k_new, a.k_new_stride_bytes);
      vnew = new_row(a.v_new, a.v_new_stride_bytes);
      const int s_last = n > 0 ? (n - 1) / a.split_tokens : 0;
      if (hc == 0 && s == s_last && lane < kCPR) {
        const uint32_t p = a.bdiv.div((uint32_t)slot_new);
        const int64_t off = (((int64_t)p * a.num_kv_heads + g) * a.bdiv.d +
                             (slot_new - p * a.bdiv.d)) * S::kRowBytes + lane * 16;
        *reinterpret_cast<u32x4*>(a.k_cache_w + off) = knew;
        *reinterpret_cast<u32x4*>(a.v_cache_w + off) = vnew;
      }
    }
  }
  if constexpr (kPrefix) {
    // splits computed once for the sequence's subgroup (after the fused
    // store above: the stored row lies past every shared split)
    const int32_t* plan = a.prefix_plan;
    if (plan[0] == a.split_tokens && plan[1] == a.prefix_items && plan[2] == a.batch &&
        plan[3] == a.group && s < plan[kPlanHeader + b])
      return;
  }
  if (start >= n) {
    if (s == 0) {  // empty context: zero output rows
      for (int i = lane; i < nh * kCPR; i += 64) {
        const int h = i / kCPR, c = i % kCPR;
        uint8_t* o = a.out + ((int64_t)b * a.num_q_heads + h0 + h) * S::kRowBytes + c * 16;
        *reinterpret_cast<u32x4*>(o) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }
  const int end = min(n, start + a.split_tokens);
  const int nsplit_b = (n + a.split_tokens - 1) / a.split_tokens;

  // query rows of the heads handled here -> LDS
  for (int i = lane; i < kHeads * kCPR; i += 64) {
    const int h = i / kCPR, c = i % kCPR;
    q_lds[i] = h < nh ? *reinterpret_cast<const u32x4*>(a.q + b * a.q_stride_bytes +
                                                         (int64_t)(h0 + h) * S::kRowBytes + c * 16)
                      : u32x4{0u, 0u, 0u, 0u};
  }

  float m[kHeads], lsum[kHeads], acc[kHeads][kVec];
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[h][e] = 0.f;
  }

  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  const int grp = lane / kCPR;  // token group of this lane in the PV layout
  const int col = lane % kCPR;  // 16-byte column of this lane in the PV layout
  const int t_row = lane % kTok;

  // Block-table entries of this split, one per lane, loaded once: a split
  // spans at most 64 blocks (the plan bounds split_tokens by the block
  // size), so the per-chunk lookup is a readlane and never a load + wait
  // inside the pipelined loop.
  const uint32_t bs = a.bdiv.d;
  const int tab_base = (int)a.bdiv.div((uint32_t)start);
  const int tab_idx = tab_base + lane;
  const int tab = tab_idx < (int)a.bdiv.div((uint32_t)(end + bs - 1)) ? table[tab_idx] : 0;
  // Byte offset of the (block, kv head g) rows starting at key c0.
  auto chunk_base = [&](int c0) -> int64_t {
    const uint32_t q = kSmall ? (uint32_t)c0 >> a.bshift : a.bdiv.div((uint32_t)c0);
    const int64_t blk = __builtin_amdgcn_readlane(tab, (int)q - tab_base);
    return ((blk * a.num_kv_heads + g) * bs + (c0 - q * bs)) * S::kRowBytes;
  };
  // Byte offset of load i of the chunk at c0 (kRowsPerLoad rows, 1 KiB).
  auto load_base = [&](int64_t cbase, int c0, int i) -> int64_t {
    if constexpr (kSmall) return chunk_base(c0 + i * S::kRowsPerLoad);
    else return cbase + i * 1024;
  };
  // The K (or V) rows of the chunk at c0 into dst.  A chunk in one block is
  // read through a buffer resource that covers only its rows inside the
  // split, so the rows past the context in a sequence's last chunk arrive
  // as zeros without being read (they are masked either way).  Blocks
  // shorter than a chunk: one lookup and one plain load per 1 KiB.  With 8
  // heads per workgroup the resource's registers would push the kernel
  // past 256 VGPRs (one wave per SIMD instead of two), so that variant
  // reads the whole chunk with plain loads.
  constexpr bool kBounded = !kSmall && kHeads <= 4;
  auto load_chunk = [&](u32x4 (&dst)[S::kLoads], const uint8_t* cache, int64_t cbase, int c0) {
    if constexpr (kBounded) {
      const __amdgpu_buffer_rsrc_t r =
          bounded_rsrc(cache + cbase, min(kTok, end - c0) * S::kRowBytes);
#pragma unroll
      for (int i = 0; i < S::kLoads; ++i) dst[i] = stream_load(r, i * 1024 + lane * 16);
    }
  };
  // position whose K/V come from the fused store's input (-1: none here)
  int p_new = -1;
  if (slot_new >= 0 && n - 1 >= start && n - 1 < end) {
    const int pos = n - 1;
    const uint32_t q = a.bdiv.div((uint32_t)pos);
    const int blk = __builtin_amdgcn_readlane(tab, (int)q - tab_base);
    if (slot_new == blk * (int)bs + (pos - (int)(q * bs))) p_new = pos;
  }

  // Software pipeline: the next chunk's K is loaded as soon as the current
  // K has been copied to LDS (reusing its registers), the next chunk's V as
  // soon as the current V has been consumed, so both loads overlap a whole
  // chunk of compute.  The last chunk is peeled so the loop body issues its
  // prefetches unconditionally (a conditional load would make the compiler
  // wait for every outstanding load at the join).
  u32x4 kr[S::kLoads], vr[S::kLoads];
  {
    const int64_t base = kSmall ? 0 : chunk_base(start);
    if constexpr (!kBounded) {
#pragma unroll
      for (int i = 0; i < S::kLoads; ++i)
        kr[i] = stream_load(a.k_cache + load_base(base, start, i) + lane * 16);
#pragma unroll
      for (int i = 0; i < S::kLoads; ++i)
        vr[i] = stream_load(a.v_cache + load_base(base, start, i) + lane * 16);
    } else {
      load_chunk(kr, a.k_cache, base, start);
      load_chunk(vr, a.v_cache, base, start);
    }
  }

  auto chunk = [&](int c0, auto prefetch_tag, int64_t next_base) {
    const int c_next = c0 + kTok;
    constexpr bool kPrefetch = decltype(prefetch_tag)::value;
    __syncthreads();  // one wavefront: orders the previous chunk's LDS reads
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      const int r = i * S::kRowsPerLoad + grp;
      k_lds[r * (kCPR + 1) + col] = kr[i];
    }
    // the fused store's row replaces the cache row (last chunk only; the
    // later LDS write of the same wave wins)
    const bool sub = !kPrefetch && p_new >= c0 && p_new < c0 + kTok;  // uniform
    if (sub && lane < kCPR)
      k_lds[(p_new - c0) * (kCPR + 1) + lane] =
          kReloadNew ? new_row(a.k_new, a.k_new_stride_bytes) : knew;
    __syncthreads();
    if constexpr (kPrefetch) {
      if constexpr (!kBounded) {
#pragma unroll
        for (int i = 0; i < S::kLoads; ++i)
          kr[i] = stream_load(a.k_cache + load_base(next_base, c_next, i) + lane * 16);
      } else {
        load_chunk(kr, a.k_cache, next_base, c_next);
      }
    }

    const int nvalid = min(kTok, end - c0);

    // scores: lane t_row owns token c0 + t_row.  q is re-read from LDS for
    // every chunk: an opaque zero offset keeps the compiler from hoisting all
    // of q (64 VGPRs per head) out of the loop.
    int qz;
    asm volatile("s_mov_b32 %0, 0" : "=s"(qz));
    const u32x4* qrow = q_lds + qz;
    float sc[kHeads];
#pragma unroll
    for (int h = 0; h < kHeads; ++h) sc[h] = 0.f;
#pragma unroll 2
    for (int c = 0; c < kCPR; ++c) {
      const u32x4 kv = k_lds[t_row * (kCPR + 1) + c];
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        const u32x4 qv = qrow[h * kCPR + c];
        if constexpr (kElemBytes == 2) {
          sc[h] = dot2_bf16(kv[0], qv[0], sc[h]);
          sc[h] = dot2_bf16(kv[1], qv[1], sc[h]);
          sc[h] = dot2_bf16(kv[2], qv[2], sc[h]);
          sc[h] = dot2_bf16(kv[3], qv[3], sc[h]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sc[h] = fmaf(__uint_as_float(kv[e]), __uint_as_float(qv[e]), sc[h]);
        }
      }
    }

    const bool tok_valid = (lane < kTok) && (t_row < nvalid);
    float x[kHeads], cmax[kHeads];
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      x[h] = tok_valid ? sc[h] * a.scale_log2 : -INFINITY;
      cmax[h] = wave_max(x[h]);
    }
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      const float mn = fmaxf(m[h], cmax[h]);  // finite: the chunk has a valid token
      const float alpha = fast_exp2(m[h] - mn);
      const float p = fast_exp2(x[h] - mn);
      lsum[h] = lsum[h] * alpha + p;
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < kVec; ++e) acc[h][e] *= alpha;
      if (lane < kTok) p_lds[t_row * kHeads + h] = p;
    }
    __syncthreads();

    if (sub) {
      const u32x4 vn = kReloadNew ? new_row(a.v_new, a.v_new_stride_bytes) : vnew;
#pragma unroll
      for (int i = 0; i < S::kLoads; ++i)
        if (i * S::kRowsPerLoad + grp == p_new - c0) vr[i] = vn;
    }
    // PV: lane holds kVec dims (column col) of tokens i*kRowsPerLoad + grp
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      const int r = i * S::kRowsPerLoad + grp;
      float vals[kVec];
      unpack<kElemBytes>(vr[i], vals);
      if (r >= nvalid) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) vals[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        const float p = p_lds[r * kHeads + h];
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[h][e] = fmaf(p, vals[e], acc[h][e]);
      }
    }
    if constexpr (kPrefetch) {
      if constexpr (!kBounded) {
#pragma unroll
        for (int i = 0; i < S::kLoads; ++i)
          vr[i] = stream_load(a.v_cache + load_base(next_base, c_next, i) + lane * 16);
      } else {
        load_chunk(vr, a.v_cache, next_base, c_next);
      }
    }
  };

  int c0 = start;
  for (; c0 + kTok < end; c0 += kTok) chunk(c0, TrueTag{}, kSmall ? 0 : chunk_base(c0 + kTok));
  chunk(c0, FalseTag{}, 0);

  // sum the token groups (lanes col, col + kCPR, ...) and the per-lane l
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
#pragma unroll
      for (int o = kCPR; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o, 64);
    }
    lsum[h] = wave_sum(lsum[h]);
  }

  if (nsplit_b == 1) {
    if (lane < kCPR) {
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        if (h >= nh) break;
        const float inv = 1.0f / lsum[h];
        uint8_t* o = a.out + ((int64_t)b * a.num_q_heads + h0 + h) * S::kRowBytes + col * 16;
        u32x4 w;
        if constexpr (kElemBytes == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = pack_bf16(acc[h][2 * i] * inv, acc[h][2 * i + 1] * inv);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(acc[h][i] * inv);
        }
        *reinterpret_cast<u32x4*>(o) = w;
      }
    }
    return;
  }

  // ---- split-K: leave this split's partials for the merge kernel ----------
  if (lane < kCPR) {
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      if (h >= nh) break;
      const int64_t slot = ((int64_t)b * a.num_q_heads + h0 + h) * a.nsplit + s;
      float* dst = a.ws_acc + slot * kHeadDim + col * kVec;
#pragma unroll
      for (int e = 0; e < kVec; e += 4)
        *reinterpret_cast<f32x4*>(dst + e) =
            f32x4{acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]};
      if (lane == 0) *reinterpret_cast<f32x2*>(a.ws_ml + slot * 2) = f32x2{m[h], lsum[h]};
    }
  }
}

// Merge the split partials of one (sequence, query head) per wavefront:
// M = max_s m_s, out = sum_s 2^(m_s-M) acc_s / sum_s 2^(m_s-M) l_s, with the
// acc sum taken in split order.  The kernel is latency-bound (a few KB per
// wavefront), so every load is issued before the first use: lane s fetches
// split s's (m, l), and the acc rows of a batch of splits (4 or 16) are in
// flight while the maximum is reduced.  Splits beyond 64 (very long
// contexts with small splits) go through the general loop.  Sequences with
// a single split were finished by the split kernel.
//
// merge_pair: one (sequence, query head) pair with ns splits, acc rows read
// kBatch at a time (rows past the end are re-reads of the last row, with
// weight 0).  kStaged (kBatch 16; decode_merge_wide_kernel): rows 16..63 of
// each group of 64 splits are not loaded here but taken from `stage`, where
// wavefronts 1-3 of the workgroup load them (merge_stage_rows) while this
// one loads rows 0..15 -- one round of loads per group instead of four, and
// the same arithmetic in the same order, so bitwise the same result.  Both
// sides pass two barriers per group: rows staged, stage free again.
template <int kElemBytes, int kBatch, bool kStaged = false>
__device__ __forceinline__ void merge_pair(const DecodeArgs& a, int pair, int ns,
                                           const f32x2 (*stage)[64] = nullptr) {
  static_assert(!kStaged || kBatch == 16, "staged rows come in batches of 16");
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)pair * a.nsplit;
  const float* acc_rows = a.ws_acc + base * kHeadDim + lane * 2;

  // first group: (m, l) of splits 0..63 and acc rows of splits 0..kBatch-1
  f32x2 ml = f32x2{-INFINITY, 0.f};
  if (lane < ns) ml = *reinterpret_cast<const f32x2*>(a.ws_ml + (base + lane) * 2);
  f32x2 v[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    v[j] = *reinterpret_cast<const f32x2*>(acc_rows + (int64_t)min(j, ns - 1) * kHeadDim);

  float M = ml[0];
  for (int g0 = 64; g0 < ns; g0 += 64) {
    const int t = g0 + lane;
    M = fmaxf(M, t < ns ? a.ws_ml[(base + t) * 2] : -INFINITY);
  }
  M = wave_max(M);

  float l_lane = 0.f, o0 = 0.f, o1 = 0.f;
  for (int g0 = 0; g0 < ns; g0 += 64) {
    if (g0 > 0) {
      const int t = g0 + lane;
      ml = t < ns ? *reinterpret_cast<const f32x2*>(a.ws_ml + (base + t) * 2)
                  : f32x2{-INFINITY, 0.f};
    }
    const float f = fast_exp2(ml[0] - M);  // 0 for lanes past the end
    l_lane = fmaf(f, ml[1], l_lane);
    const int gn = min(64, ns - g0);
    if constexpr (kStaged) __syncthreads();  // this group's rows 16.. staged
    for (int j0 = 0; j0 < gn; j0 += kBatch) {
      if (kStaged && j0 > 0) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) v[j] = stage[j0 - 16 + j][lane];
      } else if (g0 > 0 || j0 > 0) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          v[j] = *reinterpret_cast<const f32x2*>(
              acc_rows + (int64_t)(g0 + min(j0 + j, gn - 1)) * kHeadDim);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float fj = j0 + j < gn ? lane_value(f, j0 + j) : 0.f;
        o0 = fmaf(fj, v[j][0], o0);
        o1 = fmaf(fj, v[j][1], o1);
      }
    }
    if constexpr (kStaged) __syncthreads();  // stage free for the next group
  }
  const float inv = 1.0f / wave_sum(l_lane);
  constexpr int kRowBytes = kHeadDim * kElemBytes;
  if constexpr (kElemBytes == 2) {
    reinterpret_cast<uint32_t*>(a.out + (int64_t)pair * kRowBytes)[lane] =
        pack_bf16(o0 * inv, o1 * inv);
  } else {
    *reinterpret_cast<f32x2*>(a.out + (int64_t)pair * kRowBytes + lane * 8) =
        f32x2{o0 * inv, o1 * inv};
  }
}

// Wavefront w = 1..3 of a decode_merge_wide_kernel workgroup: for each group
// of 64 splits, load acc rows 16w..16w+15 (clamped to the group's last row,
// as merge_pair would) into stage[16(w-1)..], then wait while wavefront 0
// consumes them.
__device__ __forceinline__ void merge_stage_rows(const DecodeArgs& a, int pair, int ns,
                                                 f32x2 (*stage)[64]) {
  const int lane = threadIdx.x & 63;
  const int r0 = (int)(threadIdx.x >> 6) * 16;
  const float* acc_rows = a.ws_acc + (int64_t)pair * a.nsplit * kHeadDim + lane * 2;
  for (int g0 = 0; g0 < ns; g0 += 64) {
    const int gn = min(64, ns - g0);
    if (r0 < gn) {
      f32x2 v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        v[j] = *reinterpret_cast<const f32x2*>(
            acc_rows + (int64_t)(g0 + min(r0 + j, gn - 1)) * kHeadDim);
#pragma unroll
      for (int j = 0; j < 16; ++j) stage[r0 - 16 + j][lane] = v[j];
    }
    __syncthreads();  // rows staged
    __syncthreads();  // wavefront 0 has read them
  }
}

// Pairs with at most 4 splits (long splits: the 256-sequence workload's
// plan has 1-4 per sequence) take a 4-row batch: the load instructions of
// the 16-row batch (12 of them re-reads) were what bounded that merge
// (11.9 -> 8.6 us, bitwise equal; a path per power of two up to 32 cost
// registers and occupancy and was slower).  Four pairs per workgroup, one
// per wavefront.
template <int kElemBytes>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= a.batch * a.num_q_heads) return;
  const int b = pair / a.num_q_heads;
  const int n = a.context_lens[b];
  const int ns = (n + a.split_tokens - 1) / a.split_tokens;
  if (ns <= 1) return;
  if (ns <= 4)
    merge_pair<kElemBytes, 4>(a, pair, ns);
  else
    merge_pair<kElemBytes, 16>(a, pair, ns);
}

// Plans with more than 16 splits: one pair per workgroup of four
// wavefronts.  A pair with more than 16 splits is merged by wavefront 0
// with wavefronts 1-3 loading its acc rows (see merge_pair); one with fewer
// by wavefront 0 alone, exactly as decode_merge_kernel does.  (The branches
// depend only on the pair, i.e. on the workgroup, so every wavefront of a
// workgroup passes the same barriers or none.)
template <int kElemBytes>
__global__ __launch_bounds__(256) void decode_merge_wide_kernel(DecodeArgs a) {
  __shared__ f32x2 stage[48][64];
  const int pair = blockIdx.x;
  const int b = pair / a.num_q_heads;
  const int n = a.context_lens[b];
  const int ns = (n + a.split_tokens - 1) / a.split_tokens;
  if (ns <= 1) return;
  if (ns <= 16) {
    if (threadIdx.x >= 64) return;
    if (ns <= 4)
      merge_pair<kElemBytes, 4>(a, pair, ns);
    else
      merge_pair<kElemBytes, 16>(a, pair, ns);
    return;
  }
  if (threadIdx.x < 64)
    merge_pair<kElemBytes, 16, true>(a, pair, ns, stage);
  else
    merge_stage_rows(a, pair, ns, stage);
}

template <int kElemBytes, int kHeads, bool kSmall>
void launch_split_b(const DecodeArgs& args, unsigned grid, hipStream_t stream) {
  if constexpr (kElemBytes == 2) {
    if (args.prefix_plan) {
      if (args.k_new)
        hipLaunchKernelGGL((decode_split_kernel<2, kHeads, true, kSmall, true>), dim3(grid),
                           dim3(64), 0, stream, args);
      else
        hipLaunchKernelGGL((decode_split_kernel<2, kHeads, false, kSmall, true>), dim3(grid),
                           dim3(64), 0, stream, args);
      return;
    }
  }
  if (args.k_new)
    hipLaunchKernelGGL((decode_split_kernel<kElemBytes, kHeads, true, kSmall, false>), dim3(grid),
                       dim3(64), 0, stream, args);
  else
    hipLaunchKernelGGL((decode_split_kernel<kElemBytes, kHeads, false, kSmall, false>), dim3(grid),
                       dim3(64), 0, stream, args);
}

template <int kElemBytes, int kHeads>
void launch_split(const DecodeArgs& args, unsigned grid, hipStream_t stream) {
  if ((int)args.bdiv.d < DecodeShape<kElemBytes>::kTokens)
    launch_split_b<kElemBytes, kHeads, true>(args, grid, stream);
  else
    launch_split_b<kElemBytes, kHeads, false>(args, grid, stream);
}

template <int kElemBytes>
void launch_split_heads(int heads, const DecodeArgs& args, unsigned grid, hipStream_t stream) {
  switch (heads) {
    case 1: launch_split<kElemBytes, 1>(args, grid, stream); break;
    case 2: launch_split<kElemBytes, 2>(args, grid, stream); break;
    case 4: launch_split<kElemBytes, 4>(args, grid, stream); break;
    default: launch_split<kElemBytes, 8>(args, grid, stream); break;
  }
}

}  // namespace

// Query heads per workgroup: the group itself when it is 1, 2, 4 or 8;
// otherwise the next of those sizes (8 for groups above 8), the heads past
// the group masked in the last chunk -- each workgroup still reads its kv
// head's K/V once for all the heads it serves.
int decode_heads_per_wg(int group) {
  if (group < 1) return 0;
  if (group >= 8) return 8;
  int h = 1;
  while (h < group) h <<= 1;
  return h;
}

bool plan_decode(int batch, int num_q_heads, int num_kv_heads, int max_context_len,
                 int num_splits, int block_size, DecodePlan* plan) {
  const int group = num_q_heads / num_kv_heads;
  const int hpw = decode_heads_per_wg(group);
  if (hpw == 0) return false;
  plan->group = group;
  plan->heads_per_wg = hpw;
  plan->head_chunks = (group + hpw - 1) / hpw;
  const int64_t units = (int64_t)batch * num_kv_heads * plan->head_chunks;
  const int max_chunks = max_context_len > 0 ? (max_context_len + 63) / 64 : 1;
  int64_t want;
  if (num_splits > 0) {
    want = num_splits;
  } else {
    // 64-token chunks if every sequence were max_context_len long
    const int64_t chunks = units * max_chunks;
    const int64_t target =
        chunks <= (int64_t)kSmallPlanChunks * kSmallTargetWaves ? kSmallTargetWaves : kTargetWaves;
    want = units > 0 ? (target + units - 1) / units : 1;
  }
  if (want < 1) want = 1;
  if (want > max_chunks) want = max_chunks;
  const int per = max_context_len > 0 ? (int)((max_context_len + want - 1) / want) : 64;
  // Splits of up to 256 keys are multiples of 64 (a chunk starts on a
  // multiple of 64 and so never crosses a block of 64 k tokens); longer
  // splits are multiples of 256.  A split's block-table entries must fit one
  // register (64 lanes): a split aligned to the blocks spans split / B of
  // them, an unaligned one up to split / B + 2.
  int split = per <= 256 ? ((per + 63) / 64) * 64 : ((per + 255) / 256) * 256;
  const int gran = split <= 256 ? 64 : 256;
  const int64_t cap_tokens = (gran % block_size == 0 ? 64 : 62) * (int64_t)block_size;
  const int cap = (int)std::min<int64_t>(cap_tokens / gran * gran, 1 << 30);
  if (split > cap) split = cap;
  plan->split_tokens = split;
  plan->nsplit = max_context_len > 0 ? (max_context_len + plan->split_tokens - 1) / plan->split_tokens : 1;
  if (plan->nsplit > 1) {
    plan->workspace_bytes = (size_t)batch * num_q_heads * plan->nsplit * (kHeadDim + 2) * 4;
  } else {
    plan->workspace_bytes = 0;
  }
  return true;
}

static DecodeArgs decode_args(int elem_bytes, const DecodePlan& plan, const DecodeLaunch& l) {
  DecodeArgs a;
  a.q = (const uint8_t*)l.q;
  a.q_stride_bytes = l.q_stride * elem_bytes;
  a.k_cache = (const uint8_t*)l.k_cache;
  a.v_cache = (const uint8_t*)l.v_cache;
  a.block_tables = l.block_tables;
  a.max_blocks = l.max_blocks;
  a.context_lens = l.context_lens;
  a.batch = l.batch;
  a.num_q_heads = l.num_q_heads;
  a.num_kv_heads = l.num_kv_heads;
  a.group = plan.group;
  a.head_chunks = plan.head_chunks;
  a.bdiv = FastDiv((uint32_t)l.block_size);
  a.bshift = 0;
  while ((1 << a.bshift) < l.block_size) ++a.bshift;
  a.scale_log2 = l.scale * kLog2e;
  a.split_tokens = plan.split_tokens;
  a.nsplit = plan.nsplit;
  a.out = (uint8_t*)l.out;
  a.ws_acc = l.workspace;
  a.ws_ml = l.workspace
                ? l.workspace + (size_t)l.batch * l.num_q_heads * plan.nsplit * kHeadDim
                : nullptr;
  a.k_new = (const uint8_t*)l.k_new;
  a.v_new = (const uint8_t*)l.v_new;
  a.k_new_stride_bytes = l.k_new_stride * elem_bytes;
  a.v_new_stride_bytes = l.v_new_stride * elem_bytes;
  a.slot_mapping = l.slot_mapping;
  a.k_cache_w = (uint8_t*)l.k_cache;
  a.v_cache_w = (uint8_t*)l.v_cache;
  a.prefix_plan = l.prefix_plan;
  a.prefix_items = l.prefix_plan ? l.prefix_items : 0;
  a.prefix_wgs = a.prefix_items * l.num_kv_heads;
  // compacted units when several splits exist; the row walk of unit_of is
  // bounded by nsplit
  a.compact = l.batch > 1 && l.batch <= kMaxCompactBatch && plan.nsplit >= kMinCompactSplits &&
              plan.nsplit <= kMaxCompactSplits && plan.split_tokens >= kMinCompactSplit;
  a.sdiv = FastDiv((uint32_t)plan.split_tokens);
  return a;
}

hipError_t launch_decode_split(int elem_bytes, const DecodePlan& plan, const DecodeLaunch& l,
                               hipStream_t stream) {
  const DecodeArgs a = decode_args(elem_bytes, plan, l);
  const int64_t grid =
      (int64_t)plan.nsplit * l.batch * l.num_kv_heads * plan.head_chunks + a.prefix_wgs;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (elem_bytes == 2)
    launch_split_heads<2>(plan.heads_per_wg, a, (unsigned)grid, stream);
  else
    launch_split_heads<4>(plan.heads_per_wg, a, (unsigned)grid, stream);
  return hipGetLastError();
}

hipError_t launch_decode_merge(int elem_bytes, const DecodePlan& plan, const DecodeLaunch& l,
                               hipStream_t stream) {
  if (plan.nsplit <= 1 || l.batch <= 0) return hipSuccess;  // nothing was split
  const DecodeArgs a = decode_args(elem_bytes, plan, l);
  const int64_t pairs = (int64_t)l.batch * l.num_q_heads;
  if (plan.nsplit > 16) {
    if (pairs > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (elem_bytes == 2)
      hipLaunchKernelGGL(decode_merge_wide_kernel<2>, dim3((unsigned)pairs), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_merge_wide_kernel<4>, dim3((unsigned)pairs), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const unsigned mgrid = (unsigned)((pairs + 3) / 4);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(decode_merge_kernel<2>, dim3(mgrid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<4>, dim3(mgrid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
