// Varlen causal prefill over a paged, prefix-cached KV cache (gfx950, bf16).
//
// Operation (nano-vllm source study, section 2: varlen attention with prefix
// cache in prefill; architecture page, "Prefill- und Decode-Vorbereitung":
// the uncached tokens are positions num_cached_tokens .. seqlen-1, and
// "Hash-basiertes Prefix Caching": cached prefix blocks are shared whole):
// sequence b has n_q query rows (cu_seqlens_q) and n_k = context_lens[b] keys
// in the cache; query i sits at position n_k - n_q + i and attends keys
// 0 .. n_k - n_q + i, all gathered through block_tables[b].
//
// MFMA formulation.  Everything runs on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  Scores are computed transposed, S^T = K * Q^T (keys are the
// MFMA rows, queries the columns), so each lane holds 32 keys of ONE query:
// the softmax row max/sum is in-lane plus one exchange with lane l^32, and
// the probabilities come out of the accumulator already in the layout the
// next MFMA wants as its B operand.  Output is accumulated transposed too,
// O^T += V^T * P^T; the V^T operand is read straight from the natural V tile
// with the LDS transpose read (ds_read_b64_tr_b16).
//
// Work decomposition.  A work item is 8 wavefronts x 32 query rows of one
// kv head g of one sequence: 4 query heads of g's group x 64 positions
// (group a multiple of 4), 2 heads x 128 positions (other even groups) or
// 1 head x 256 positions (odd groups).  All 8 waves share every K/V tile the
// workgroup stages.  Keys
// are processed in tiles of 64 (a tile never crosses a 256-token block, so
// one block-table entry per tile; the item's entries are loaded once).
// Items are numbered last-query-tile first (most keys first) and handed
// out by a persistent kernel (one workgroup per CU) from per-XCD queues, so
// the items of one (sequence, kv head) share one L2.
//
// Schedule.  The 8 waves form two groups of 4 (one wave of each group per
// SIMD); every tile is an MFMA phase (S of this tile, PV of the previous
// one, at raised wave priority) and a softmax phase, with group B one phase
// behind group A and a workgroup barrier between phases.  Group A copies K and V tiles global ->
// LDS with the direct-to-LDS buffer load (no registers, no VALU) two tiles
// ahead into 4 rotating slots (128 KiB of LDS).  The buffer resource of a
// copy covers only the tile's rows inside the context, so rows past it
// arrive as zeros.
//
// Softmax work per tile is kept small because it competes with the MFMAs
// for issue slots: the causal mask is a select, the scale is folded into
// the exponent's FMA, and the row max (and the rescaling of O) is only
// computed on tiles whose probabilities against the current running max
// would exceed 2^16 (lazy rescaling); the row sums use v_dot2 on the packed
// bf16 probabilities.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kQT = 32;          // query rows per wave
constexpr int kKT = 64;          // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kGroupWaves = 4;   // waves per ping-pong group
constexpr int kSlots = 4;        // LDS slots for K and for V tiles
constexpr int kAhead = 2;        // tiles copied ahead of the phase that first reads them
constexpr int kCopyOps = 8;      // direct-to-LDS loads per group-A wave per tile (K 4, V 4)
constexpr int kMaxQueues = 8;    // one per XCD

struct PrefillArgs {
  const uint16_t* q;
  int64_t q_stride;  // elements
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* cu_q;
  const int32_t* ctx;
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t batch, num_q_heads, num_kv_heads, group;
  int32_t heads_per_wg, pos_tiles, head_chunks, max_wg_tiles;
  float scale_log2;  // |scale| * log2(e), or log2(e) for a zero scale (> 0 either way)
  // Applied to every 32-bit word (two bf16) of q: (word & q_keep) ^ q_flip.
  // The kernel masks scores to -inf before scaling, which needs a positive
  // scale; scale * q.k is computed exactly as |scale| * (-q).k for a
  // negative scale (a sign flip of a bf16 is exact) and as 1 * (0 . k) for
  // a zero one.
  uint32_t q_keep, q_flip;
  uint16_t* out;
  // Keys from contiguous rows instead of the cache (no block table):
  // sequence b's keys are rows cu_k[b] .. cu_k[b+1]-1 of k_rows / v_rows.
  // cu_k == nullptr: keys come from the cache through block_tables.
  const int32_t* cu_k;
  const uint16_t* k_rows;
  const uint16_t* v_rows;
  int64_t k_row_stride, v_row_stride;  // elements between key rows
  FastDiv bdiv;  // cache block size (bdiv.d) and division by it
  int32_t num_items;   // work items: (query tile, sequence, kv head, head chunk)
  int32_t num_queues;  // work queues (one per XCD when the grid allows)
  int32_t* counters;   // [kMaxQueues] queue heads, then the exit count
};

// Bound on the probabilities computed against a lagging running max (see
// the softmax step): with p <= 2^16, O and l stay far inside fp32 range
// for any context the cache can hold.
constexpr float kLazyBound = 65536.0f;
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// K and V tiles live in LDS in their natural [64 keys][128 dims] bf16 order,
// 256 bytes per key row, with the 16-byte chunks of row `key` permuted:
//   K: chunk c at position c ^ (key & 15)
//   V: chunk c at position c ^ (4 * (key & 3))   (64-byte blocks permuted)
// so that the MFMA operand reads below hit distinct LDS banks.  (For V the
// transpose reads of one instruction cover 8 keys x 8 dim groups; with the
// permutation the 32 lanes of each half wave address 32 distinct 8-byte
// bank pairs -- rocprofv3 SQ_LDS_BANK_CONFLICT reads 0.)  Tiles are
// copied global -> LDS by the direct-to-LDS load (no registers, no VALU):
// lane l of a wave instruction lands at LDS base + 16 l, so each lane fetches
// the global chunk that belongs at that position.
__device__ __forceinline__ int k_pos(int key, int c) { return c ^ (key & 15); }
__device__ __forceinline__ int v_pos(int key, int c) { return c ^ ((key & 3) << 2); }

// Copy one 64-key tile (K or V) into LDS: each of the 4 group-A waves moves
// 16 keys, 1 KiB per instruction.  The per-lane byte offsets depend only on
// the lane and wave, so they are computed once (tile_offsets) and a new tile
// only changes the scalar buffer base.  With cache blocks of a multiple of 64
// tokens a tile lies in one block and one resource (base row k0) serves the
// 4 waves (`wave` = the wave's index in its group).  With blocks of 16 or 32
// tokens a tile spans several blocks; each wave's 16 rows still lie in one,
// so each wave uses its own resource based at its first row (`wave` = 0).
// The swizzle uses key & 15, the same either way.
template <bool kIsV>
__device__ __forceinline__ void tile_offsets(uint32_t (&voff)[4], int wave, int lane,
                                             uint32_t row_bytes) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = wave * 16 + i * 4 + (lane >> 4);
    const int pos = lane & 15;
    const int c = kIsV ? v_pos(key, pos) : k_pos(key, pos);  // the involution maps back
    voff[i] = (uint32_t)key * row_bytes + (uint32_t)c * 16u;
  }
}

__device__ __forceinline__ void tile_to_lds(__amdgpu_buffer_rsrc_t rsrc, const uint32_t (&voff)[4],
                                            u32x4* lds, int wave) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + (wave * 16 + i * 4) * 16), 16,
                                             voff[i], 0, 0, 0);
}

// Raw buffer resource over the valid rows of one K or V tile (word 3:
// 32-bit data format, the value used for untyped buffer access on
// gfx9-family parts).  Loads past `bytes` return zero, so the rows of a
// tile that lie past the context arrive in LDS as zeros: masked
// probabilities are 0 and 0 * 0 stays 0 in the PV product.
//
// Every argument is the same in all lanes of the wave, but when it was
// computed under a branch on the wave index (only group A copies) the
// compiler cannot prove that and would wrap each copy in a loop over the
// distinct resources of the lanes; readfirstlane states the uniformity.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), 0,
      __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8).
template <int kVm>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(kVm >= 0 && kVm < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | kVm);
}

// Barrier between phases.  No memory fence: copies issued for later tiles
// stay in flight (their completion is awaited explicitly with vmcnt).  This
// wave's LDS accesses complete first, and the compiler may not move memory
// accesses across it.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One work item: query tile r (counted from the end) of sequence b, kv head
// g, head chunk hc, on 8 waves in two groups of 4 (see the kernel).
// kBlock: the cache block size when it is fixed at compile time (a power of
// two from 64 to 4096, 256 being the pages' size: divisions become shifts),
// 0 for any other multiple of 64 (division by multiplication), -1 for
// blocks of 16 or 32 tokens (see tile_offsets).
template <int kBlock>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, int id, u32x4 (*kbuf)[kKT * 16],
                                             u32x4 (*vbuf)[kKT * 16]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 31;  // query column / MFMA row index
  const int hf = lane >> 5;
  const bool group_a = wave < kGroupWaves;

  const int hc = id % a.head_chunks;
  id /= a.head_chunks;
  const int g = id % a.num_kv_heads;
  id /= a.num_kv_heads;
  const int b = id % a.batch;
  const int r = id / a.batch;  // workgroup tile counted from the end

  // Block-table entries of the item, loaded once: lane i holds logical
  // blocks i and 64 + i; beyond 128 blocks a scalar load (constant address
  // space) is used.  A per-tile global load would make the copy wait on
  // every vector memory access in flight, including the copies of the
  // previous tiles.  The row's first 128 columns are loaded whether the
  // item uses them or not (all inside the table), before the sequence's
  // lengths are known, so that the two loads share one memory round trip.
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  const int tcols = (a.cu_k || !a.block_tables) ? 0 : min(a.max_blocks, 128);
  const int32_t tab0 = lane < tcols ? table[lane] : 0;
  const int32_t tab1 = lane + 64 < tcols ? table[lane + 64] : 0;

  // The sequence's lengths: uniform over the workgroup and read-only for the
  // launch, so scalar loads (constant address space) through the scalar
  // cache, which every item of the launch shares; as plain loads they were
  // vector loads, each waited for in turn.
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  auto sload = [](const int32_t* p, int i) { return ((const_i32*)p)[i]; };
  const int q_begin = sload(a.cu_q, b);
  const int n_q = sload(a.cu_q, b + 1) - q_begin;
  const int k_begin = a.cu_k ? sload(a.cu_k, b) : 0;
  const int n_k = a.cu_k ? sload(a.cu_k, b + 1) - k_begin : sload(a.ctx, b);
  const int off = n_k - n_q;
  const int wg_rows = kQT * a.pos_tiles;
  const int wg_tiles = (n_q + wg_rows - 1) / wg_rows;
  if (r >= wg_tiles) return;  // uniform over the workgroup, before any barrier
  const int wg_q0 = (wg_tiles - 1 - r) * wg_rows;

  const int my_q0 = wg_q0 + (wave / a.heads_per_wg) * kQT;
  const int h = g * a.group + hc * a.heads_per_wg + (wave % a.heads_per_wg);
  const bool wave_has_rows = my_q0 < n_q;
  // keys seen by the last query of the workgroup / of this wave
  const int wg_kend = max(0, min(n_k, off + min(n_q, wg_q0 + wg_rows)));
  const int my_kend = wave_has_rows ? max(0, min(n_k, off + min(n_q, my_q0 + kQT))) : 0;
  const int ntiles = (wg_kend + kKT - 1) / kKT;
  const int my_tiles = (my_kend + kKT - 1) / kKT;

  // this lane's query column: row qi of the sequence (clamped for loads)
  const int qi = my_q0 + j;
  const int q_pos = off + qi;  // last visible key of this query
  u32x4 qreg[8];
  {
    const int q_row = q_begin + min(qi, max(n_q - 1, 0));
    const uint16_t* qp = a.q + (int64_t)q_row * a.q_stride + (int64_t)h * kHeadDim + hf * 8;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qp + kb * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) qreg[kb][e] = (w[e] & a.q_keep) ^ a.q_flip;
    }
  }

  f32x16 o_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o_acc[db] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;
  const float c = a.scale_log2;

  constexpr bool kSmall = kBlock < 0;
  const uint32_t bs = kBlock > 0 ? (uint32_t)kBlock : a.bdiv.d;
  auto block_of = [&](uint32_t key) -> uint32_t {
    if constexpr (kBlock > 0) return key / (uint32_t)kBlock;
    else if constexpr (kSmall) return key >> (bs == 16 ? 4 : 5);
    else return a.bdiv.div(key);
  };
  auto block_at = [&](int i) -> int64_t {  // i uniform
    if (i < 64) return __builtin_amdgcn_readlane(tab0, i);
    if (i < 128) return __builtin_amdgcn_readlane(tab1, i - 64);
    return ((const __attribute__((address_space(4))) int32_t*)table)[i];
  };
  // key rows of a tile are 256 bytes apart in the cache, a token stride apart
  // in contiguous k / v
  const uint32_t k_row_bytes = a.cu_k ? (uint32_t)(a.k_row_stride * 2) : kHeadDim * 2;
  const uint32_t v_row_bytes = a.cu_k ? (uint32_t)(a.v_row_stride * 2) : kHeadDim * 2;
  uint32_t k_off[4], v_off[4];
  const int gw = kSmall ? 0 : (wave & (kGroupWaves - 1));
  tile_offsets<false>(k_off, gw, lane, k_row_bytes);
  tile_offsets<true>(v_off, gw, lane, v_row_bytes);
  // kBlock == 0: the copies run over the tiles in order, so the tile's
  // (block index, row in block) advances by one tile per call instead of
  // being divided out
  uint32_t cp_blk = 0, cp_row = 0;
  auto issue_copy = [&](int t) {  // group A only, t = 0, 1, 2, ... in order
    const int k0 = t * kKT;
    const int nvalid = min(kKT, n_k - k0);
    const uint16_t *kb, *vb;
    int nbytes_k, nbytes_v;
    if constexpr (!kSmall) {
      if (a.cu_k) {
        kb = a.k_rows + (int64_t)(k_begin + k0) * a.k_row_stride + g * kHeadDim;
        vb = a.v_rows + (int64_t)(k_begin + k0) * a.v_row_stride + g * kHeadDim;
      } else {
        uint32_t qb, row;
        if constexpr (kBlock > 0) {
          qb = block_of((uint32_t)k0);
          row = k0 - qb * bs;
        } else {
          // uniform (see tile_rsrc): a lane-varying index would turn the
          // table lookup into a vector load whose wait also waits for
          // every copy still in flight
          qb = __builtin_amdgcn_readfirstlane(cp_blk);
          row = __builtin_amdgcn_readfirstlane(cp_row);
          cp_row = row + kKT;
          cp_blk = qb;
          if (cp_row == bs) cp_row = 0, ++cp_blk;
        }
        const int64_t blk = block_at((int)qb);
        const int64_t base = ((blk * a.num_kv_heads + g) * bs + row) * kHeadDim;
        kb = a.k_cache + base;
        vb = a.v_cache + base;
      }
      nbytes_k = nvalid * (int)k_row_bytes;
      nbytes_v = nvalid * (int)v_row_bytes;
    } else {
      // this wave's 16 keys kw .. kw+15 lie in one block; keys at or past
      // wg_kend are seen by no query of the workgroup, arrive as zeros
      // (outside the resource) and need no (possibly unloaded) table entry
      const int kw = k0 + __builtin_amdgcn_readfirstlane((wave & (kGroupWaves - 1)) * 16);
      const int nv = max(0, min(16, wg_kend - kw));
      const uint32_t qb = nv > 0 ? block_of((uint32_t)kw) : 0u;
      const int64_t blk = nv > 0 ? block_at((int)qb) : 0;
      const int64_t base = ((blk * a.num_kv_heads + g) * bs + (kw - qb * bs)) * kHeadDim;
      kb = a.k_cache + base;
      vb = a.v_cache + base;
      nbytes_k = nbytes_v = nv * kHeadDim * 2;
    }
    const int slot = t % kSlots;
    tile_to_lds(tile_rsrc(kb, nbytes_k), k_off, kbuf[slot], wave);
    tile_to_lds(tile_rsrc(vb, nbytes_v), v_off, vbuf[slot], wave);
  };

  // PV operand reads (ds_read_b64_tr_b16): in each 16-lane group, lane
  // 4a+e receives element e of the 8-byte chunks addressed by lanes a, a+4,
  // a+8, a+12.  Lane (G = lane/16, a = lane%4, m = (lane%16)/4) therefore
  // addresses key kt*32 + 16ks + 4hf + m (+8 for the second half) at dims
  // 32db + 16(G%2) + 4a: the lane then holds, for dim 32db + lane%32, the
  // four keys in the order the S^T accumulator produced the probabilities.
  const int tr_g = lane >> 4;
  const int tr_a = lane & 3;
  const int tr_m = (lane >> 2) & 3;
  auto tr_read = [&](const u32x4* vb, int key, int dim) -> uint64_t {
    const int cpos = v_pos(key, dim >> 3);
    const char* p = reinterpret_cast<const char*>(vb) + key * 256 + cpos * 16 + (dim & 7) * 2;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    return __builtin_bit_cast(uint64_t, v);
  };

  f32x16 s_acc[2];
  u32x4 pfrag[4];  // B operands of the PV product: (kt, ks) -> 16 keys

  // ---- S^T = K Q^T for the 64 keys of tile t --------------------------------
  // MFMA i = (kb, kt) = (i / 2, i % 2).  The operand reads run six MFMAs
  // ahead in a fixed order, fenced by sched_barrier: left to the scheduler,
  // the read-ahead came and went with unrelated source changes (and with it
  // an lgkmcnt(0) wait before every MFMA).
  auto scores = [&](int t) {
    const u32x4* kb_ = kbuf[t % kSlots];
    constexpr int kAheadS = 6;
    u32x4 opnd[16];
    auto rd = [&](int i) {
      const int kb = i >> 1, kt = i & 1;
      const int key = kt * 32 + j;
      opnd[i] = kb_[key * 16 + k_pos(key, kb * 2 + hf)];
    };
#pragma unroll
    for (int i = 0; i < kAheadS; ++i) rd(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kb = i >> 1, kt = i & 1;
      s_acc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          as_bf16x8(opnd[i]), as_bf16x8(qreg[kb]), kb == 0 ? f32x16{} : s_acc[kt], 0, 0, 0);
      if (i + kAheadS < 16) rd(i + kAheadS);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- online softmax (base 2) of tile t -> pfrag --------------------------
  auto softmax = [&](int t) {
    const int k0 = t * kKT;
    // element e = rr*4 + ee of s_acc[kt] is key k0 + kt*32 + 8*rr + 4*hf + ee
    if ((k0 + kKT - 1 > off + my_q0) || (k0 + kKT > n_k)) {
      // masked keys (past the query's position or the context) -> -inf
      const int lim = min(q_pos, n_k - 1) - k0 - 4 * hf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ko = kt * 32 + 8 * (e >> 2) + (e & 3);
          s_acc[kt][e] = ko <= lim ? s_acc[kt][e] : -INFINITY;
        }
    }
    // Probabilities against the running max m_run (log2 units).  The row
    // max is only computed when it is needed: while every p of this tile is
    // at most 2^kLazyBound (checked through the row sum, since p >= 0) the
    // reference m_run may lag the true max -- softmax is invariant to it --
    // and O, l need no rescaling.  Otherwise (or on a query's first visible
    // tile) m_run moves to the true running max and the tile is redone.
    float psum;
    auto probs = [&](float neg_m) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(s_acc[kt][ks * 8 + e], c, neg_m));
          const u32x4 f = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                                pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
          pfrag[kt * 2 + ks] = f;
          // row sum of the bf16 probabilities the PV product consumes
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[w] = dot2_bf16(f[w], kOnesBf16x2, acc[w]);
        }
      psum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    };
    bool rebase = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    if (!rebase) {
      probs(-m_run);
      rebase = __builtin_amdgcn_ballot_w64(!(psum <= kLazyBound)) != 0;
    }
    if (rebase) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; e += 2) tmax = fmaxf(tmax, fmaxf(s_acc[kt][e], s_acc[kt][e + 1]));
      // both lane halves hold the same query: combine lanes l and l ^ 32
      const u32x2 sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, tmax),
                                                        __builtin_bit_cast(uint32_t, tmax), false, false);
      tmax = fmaxf(__builtin_bit_cast(float, sw[0]), __builtin_bit_cast(float, sw[1])) * c;
      const float m_new = fmaxf(m_run, tmax);
      // alpha = 0 when leaving -inf; 1 while the query has seen no key yet
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o_acc[db] *= alpha;
      probs(m_new == -INFINITY ? 0.f : -m_new);
    }
    l_part += psum;
  };

  // ---- O^T += V^T P^T for tile t ---------------------------------------------
  // MFMA i = (db, kt, ks) = (i / 4, (i / 2) % 2, i % 2); its A operand is two
  // transpose reads.  The reads run five MFMAs ahead in a fixed order, as in
  // the scores above.
  auto pv = [&](int t) {
    const u32x4* vb = vbuf[t % kSlots];
    constexpr int kAheadP = 5;
    u32x4 opnd[16];
    auto rd = [&](int i) {
      const int db = i >> 2, kt = (i >> 1) & 1, ks = i & 1;
      const int dim = db * 32 + 16 * (tr_g & 1) + 4 * tr_a;
      const int key = kt * 32 + ks * 16 + 4 * hf + tr_m;
      const uint64_t lo = tr_read(vb, key, dim);
      const uint64_t hi = tr_read(vb, key + 8, dim);
      opnd[i] = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
    };
#pragma unroll
    for (int i = 0; i < kAheadP; ++i) rd(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int db = i >> 2, kt = (i >> 1) & 1, ks = i & 1;
      o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          as_bf16x8(opnd[i]), as_bf16x8(pfrag[kt * 2 + ks]), o_acc[db], 0, 0, 0);
      if (i + kAheadP < 16) rd(i + kAheadP);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- ping-pong schedule ------------------------------------------------------
  // Each tile t is an MFMA phase M(t) = {S(t), PV(t-1)} followed by a VALU
  // phase V(t) = softmax(t).  Group B runs one phase behind group A, and
  // every phase ends in a workgroup barrier, so while the waves of one group
  // issue MFMAs the waves of the other (on the same SIMDs) run the softmax.
  // Group A copies tile t+2 at the start of V(t) (slots rotate over 4 tiles:
  // K(t) is last read by B in M(t), V(t) by B in M(t+1), so the slot of tile
  // t-2 is free once V(t-1) has ended); before the barrier that ends V(t) it
  // waits for its copies of tile t+1.
  if (group_a) {
    if (ntiles > 0) issue_copy(0);
    if (ntiles > 1) {
      issue_copy(1);
      wait_vmcnt<kCopyOps>();
    } else {
      wait_vmcnt<0>();
    }
  }
  phase_barrier();
  if (!group_a) phase_barrier();  // B starts one phase behind
  for (int t = 0; t < ntiles; ++t) {
    // The MFMA phase runs at raised wave priority, so that on each SIMD the
    // issue arbiter prefers the MFMAs (and their operand reads) over the
    // other group's softmax VALU (measured: 2-3 % faster, bitwise equal).
    // S(t) goes first, so its results have settled when the softmax reads
    // them after the barrier.
    __builtin_amdgcn_s_setprio(3);
    if (t < my_tiles) scores(t);
    if (t >= 1 && t - 1 < my_tiles) pv(t - 1);
    phase_barrier();
    __builtin_amdgcn_s_setprio(0);
    // copies are issued before the softmax: the next MFMA phase's first
    // operand read waits for them (the compiler cannot tell their LDS slot
    // from the one it reads), so they get the softmax's time to land
    if (group_a && t + kAhead < ntiles) issue_copy(t + kAhead);
    if (t < my_tiles) softmax(t);
    if (group_a) {
      if (t + kAhead < ntiles) wait_vmcnt<kCopyOps>();
      else wait_vmcnt<0>();
    }
    phase_barrier();
  }
  if (ntiles >= 1 && ntiles - 1 < my_tiles) pv(ntiles - 1);
  if (group_a) phase_barrier();  // matches B's extra barrier at the start

  // ---- epilogue: out[q_row][h][d] = O^T[d][j] / l ---------------------------
  if (!wave_has_rows || qi >= n_q) return;
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  uint16_t* op = a.out + ((int64_t)(q_begin + qi) * a.num_q_heads + h) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d = db * 32 + 8 * rr + 4 * hf;
      const u32x2 w = u32x2{pack_bf16(o_acc[db][rr * 4] * inv, o_acc[db][rr * 4 + 1] * inv),
                            pack_bf16(o_acc[db][rr * 4 + 2] * inv, o_acc[db][rr * 4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + d) = w;
    }
}

// Persistent kernel: one workgroup of 8 waves per CU pulls work items from
// num_queues atomic queues, longest item first.  Queue x holds items x,
// x + num_queues, ...; workgroup w starts on queue w % num_queues, so with
// the round-robin placement of workgroups on the 8 XCDs the items of one
// (sequence, kv head) run on one XCD and share its L2.  A workgroup whose
// queue is exhausted moves on to the next queue, so no XCD idles while
// another still has items.  Dynamic pulling keeps every workgroup busy
// however unequal the items are (the hardware dispatcher leaves slots idle
// when workgroup lengths vary).  The last workgroup to leave resets the
// counters, so the workspace is zero again when the kernel ends.
template <int kBlock>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
  // K and V tiles, 4 slots each (128 KiB).
  __shared__ u32x4 kbuf[kSlots][kKT * 16];
  __shared__ u32x4 vbuf[kSlots][kKT * 16];
  __shared__ int next_item[2];

  const int nq = a.num_queues;
  // queue state, used by thread 0 only
  int queue = blockIdx.x % nq;
  int exhausted = 0;  // queues found empty so far
  // blocking pull: the next item, or -1 once every queue is exhausted
  // A workspace that was not zero before the first call holds arbitrary
  // counters: an id outside [0, num_items) then counts as an exhausted queue,
  // so such a call computes wrong rows but never indexes past the problem.
  auto pull = [&]() -> int {
    while (exhausted < nq) {
      const int ticket = atomicAdd(&a.counters[queue], 1);
      const int64_t id = queue + (int64_t)ticket * nq;
      if (ticket >= 0 && id < a.num_items) return (int)id;
      queue = queue + 1 == nq ? 0 : queue + 1;
      ++exhausted;
    }
    return -1;
  };

  if (threadIdx.x == 0) next_item[0] = pull();
  phase_barrier();
  for (int it = 0;; ++it) {
    // uniform over the workgroup; readfirstlane lets the compiler keep the
    // item's indices (and the block-table entries) in scalar registers
    const int id = __builtin_amdgcn_readfirstlane(next_item[it & 1]);
    if (id < 0) break;
    prefill_item<kBlock>(a, id, kbuf, vbuf);
    // Alternating slots: thread 0 cannot rewrite a slot before every thread
    // has passed the barrier below, i.e. has read it.
    if (threadIdx.x == 0) next_item[(it + 1) & 1] = pull();
    phase_barrier();
  }
  if (threadIdx.x == 0) {
    // acq_rel: this workgroup's queue increments are ordered before its exit
    // count, so the last one out sees every increment and may clear them.
    const int done = __hip_atomic_fetch_add(&a.counters[kMaxQueues], 1, __ATOMIC_ACQ_REL,
                                            __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - 1) {
      for (int q = 0; q <= kMaxQueues; ++q)
        __hip_atomic_store(&a.counters[q], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

bool prefill_supported_group(int group) { return group >= 1; }

// CUs of the current device, cached per device (the grid of the persistent
// kernel is one workgroup per CU).
static hipError_t compute_units(int* cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) { *cus = c; return hipSuccess; }
  }
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*cus <= 0) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < 64) cache[dev].store(*cus, std::memory_order_relaxed);
  return hipSuccess;
}

hipError_t launch_prefill(const PrefillLaunch& l, hipStream_t stream) {
  PrefillArgs a;
  a.q = (const uint16_t*)l.q;
  a.q_stride = l.q_stride;
  a.k_cache = (const uint16_t*)l.k_cache;
  a.v_cache = (const uint16_t*)l.v_cache;
  a.cu_q = l.cu_seqlens_q;
  a.ctx = l.context_lens;
  a.block_tables = l.block_tables;
  a.max_blocks = l.max_blocks;
  a.batch = l.batch;
  a.num_q_heads = l.num_q_heads;
  a.num_kv_heads = l.num_kv_heads;
  a.group = l.num_q_heads / l.num_kv_heads;
  // the largest of 4, 2, 1 that divides the group
  a.heads_per_wg = a.group % 4 == 0 ? 4 : a.group % 2 == 0 ? 2 : 1;
  a.pos_tiles = kWaves / a.heads_per_wg;
  a.head_chunks = a.group / a.heads_per_wg;
  const int wg_rows = kQT * a.pos_tiles;
  a.max_wg_tiles = (l.max_seqlen_q + wg_rows - 1) / wg_rows;
  a.scale_log2 = (l.scale == 0.f ? 1.f : fabsf(l.scale)) * kLog2e;
  a.q_keep = l.scale == 0.f ? 0u : 0xFFFFFFFFu;
  a.q_flip = l.scale < 0.f ? 0x80008000u : 0u;
  a.out = (uint16_t*)l.out;
  const int64_t items = (int64_t)a.max_wg_tiles * l.batch * l.num_kv_heads * a.head_chunks;
  if (items <= 0) return hipSuccess;
  if (items > (1 << 30)) return hipErrorInvalidConfiguration;
  int cus = 0;
  hipError_t e = compute_units(&cus);
  if (e != hipSuccess) return e;
  const int grid = (int)std::min<int64_t>(items, (int64_t)cus);
  a.num_items = (int32_t)items;
  a.num_queues = std::min(grid, kMaxQueues);
  a.counters = (int32_t*)l.workspace;
  a.cu_k = l.cu_seqlens_k;
  a.k_rows = (const uint16_t*)l.k_rows;
  a.v_rows = (const uint16_t*)l.v_rows;
  a.k_row_stride = l.k_row_stride;
  a.v_row_stride = l.v_row_stride;
  a.bdiv = FastDiv((uint32_t)l.block_size);
  // Power-of-two block sizes are compile-time constants (divisions become
  // shifts); the runtime-size instantiation (kBlock = 0) serves the other
  // multiples of 64.
  const dim3 g((unsigned)grid), t(kThreads);
  if (a.cu_k) {  // contiguous keys use no block
    hipLaunchKernelGGL(prefill_kernel<kBlockSize>, g, t, 0, stream, a);
  } else {
    switch (l.block_size) {
      case 16:
      case 32: hipLaunchKernelGGL(prefill_kernel<-1>, g, t, 0, stream, a); break;
      case 64: hipLaunchKernelGGL(prefill_kernel<64>, g, t, 0, stream, a); break;
      case 128: hipLaunchKernelGGL(prefill_kernel<128>, g, t, 0, stream, a); break;
      case 256: hipLaunchKernelGGL(prefill_kernel<256>, g, t, 0, stream, a); break;
      case 512: hipLaunchKernelGGL(prefill_kernel<512>, g, t, 0, stream, a); break;
      case 1024: hipLaunchKernelGGL(prefill_kernel<1024>, g, t, 0, stream, a); break;
      case 2048: hipLaunchKernelGGL(prefill_kernel<2048>, g, t, 0, stream, a); break;
      case 4096: hipLaunchKernelGGL(prefill_kernel<4096>, g, t, 0, stream, a); break;
      default: hipLaunchKernelGGL(prefill_kernel<0>, g, t, 0, stream, a); break;
    }
  }
  return hipGetLastError();
}

size_t prefill_workspace_bytes() { return (kMaxQueues + 1) * sizeof(int32_t); }

}  // namespace pkv
