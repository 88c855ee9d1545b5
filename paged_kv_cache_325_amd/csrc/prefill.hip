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
// O^T += V^T * P^T, with V^T staged in LDS.
//
// Work decomposition.  A workgroup is 4 wavefronts and owns one kv head g of
// one sequence and 4 "query tiles" of 32 rows: 4 query heads of g's group
// at the same 32 positions (group >= 4), or 2 heads x 64 positions (group 2),
// or 1 head x 128 positions (group 1).  The 4 waves share every K/V tile the
// workgroup stages, so each K/V byte is fetched once per 128 query rows.
// Keys are processed in tiles of 64 (a tile never crosses a 256-token block,
// so one block-table lookup per tile), with the next tile prefetched into
// registers while the current one is consumed.  Workgroups are ordered
// last-query-tile first (most keys first), and consecutive workgroup ids
// differ in kv head, so with 8 kv heads all tiles of one (sequence, kv head)
// land on the same XCD and share its L2.
//
// LDS: K tile [64 keys][16 x 16 B], column c of key r at c ^ (r & 15);
//      V^T tile [128 dims][64 keys] with a key order and swizzle described
//      at vt_offset.  Both layouts keep the MFMA operand reads and the
//      staging writes free of LDS bank conflicts.  32 KiB per workgroup.
//
// Softmax work per tile is kept small because it competes with the MFMAs
// for issue slots: the causal mask is a select, the scale is folded into
// the exponent's FMA, and O is only rescaled when some query's running max
// grows by more than 2^8 (lazy rescaling).
#include <math.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

// 32-query column blocks per wave.  One block (two waves per SIMD) measured
// faster than two (one wave per SIMD, accumulators spilling into AGPR moves).
constexpr int kWaveCB = 1;
constexpr int kKT = 64;                  // keys per tile
constexpr int kThreads = 256;

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
  float scale_log2;
  uint16_t* out;
};

constexpr float kRescaleSlack = 8.0f;  // log2 units

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// V^T tile in LDS: 128 rows (dims) x 64 keys of bf16, 128 bytes per row, in
// 8-byte units.  Keys are stored so that the 8 keys one lane feeds to a PV
// MFMA -- kt*32 + 16ks + 4hf + {0..3} and the same + 8, the order in which
// the S^T accumulator hands out probabilities -- are 16 contiguous bytes:
// within each 16-key group the two bits above the 4-key group are swapped.
// The 16-byte column is XOR-swizzled with ((d >> 1) + (d >> 4)) & 7, which
// (with the staging lane map) keeps both the b64 writes and the b128 reads
// free of bank conflicts.
__device__ __forceinline__ int vt_swizzle(int d) { return ((d >> 1) + (d >> 4)) & 7; }
// 8-byte slot of the 4-key group q (keys 4q .. 4q+3) in row d
__device__ __forceinline__ int vt_offset(int d, int q) {
  const int qp = (q & ~3) | ((q & 1) << 1) | ((q >> 1) & 1);
  return d * 16 + (((qp >> 1) ^ vt_swizzle(d)) << 1) + (qp & 1);
}
// first 8-byte slot of the (permuted) 16-byte chunk c16 of row d
__device__ __forceinline__ int vt_offset_chunk(int d, int c16) {
  return d * 16 + ((c16 ^ vt_swizzle(d)) << 1);
}

// kCB column blocks of 32 queries per wave (64 queries for kCB = 2): the
// K and V^T operands read from LDS are shared by the column blocks, and one
// block's softmax (VALU) can overlap the other block's MFMAs.
template <int kCB>
__global__ __launch_bounds__(kThreads, kCB == 1 ? 2 : 1) void prefill_kernel(PrefillArgs a) {
  constexpr int kQT = 32 * kCB;  // query rows per wave
  __shared__ u32x4 k_lds[kKT * 16];      // 16 KiB
  __shared__ __attribute__((aligned(16))) u32x2 vt_lds[kHeadDim * 16];  // 16 KiB

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 31;  // query column / MFMA row index
  const int hf = lane >> 5;

  int id = blockIdx.x;
  const int hc = id % a.head_chunks;
  id /= a.head_chunks;
  const int g = id % a.num_kv_heads;
  id /= a.num_kv_heads;
  const int b = id % a.batch;
  const int r = id / a.batch;  // workgroup tile counted from the end

  const int q_begin = a.cu_q[b];
  const int n_q = a.cu_q[b + 1] - q_begin;
  const int n_k = a.ctx[b];
  const int off = n_k - n_q;
  const int wg_rows = kQT * a.pos_tiles;
  const int wg_tiles = (n_q + wg_rows - 1) / wg_rows;
  if (r >= wg_tiles) return;  // uniform over the workgroup
  const int wg_q0 = (wg_tiles - 1 - r) * wg_rows;

  const int my_q0 = wg_q0 + (wave / a.heads_per_wg) * kQT;
  const int h = g * a.group + hc * a.heads_per_wg + (wave % a.heads_per_wg);
  const bool wave_has_rows = my_q0 < n_q;
  // keys seen by the last query of the workgroup / of this wave
  const int wg_kend = max(0, min(n_k, off + min(n_q, wg_q0 + wg_rows)));
  const int my_kend = max(0, min(n_k, off + min(n_q, my_q0 + kQT)));
  const int ntiles = (wg_kend + kKT - 1) / kKT;

  // this lane's query column in block cb: row qi[cb] (clamped for loads)
  int qi[kCB], q_pos[kCB];
  u32x4 qreg[kCB][8];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    qi[cb] = my_q0 + cb * 32 + j;
    q_pos[cb] = off + qi[cb];  // last visible key of this query
    const int q_row = q_begin + min(qi[cb], max(n_q - 1, 0));
    const uint16_t* qp = a.q + (int64_t)q_row * a.q_stride + (int64_t)h * kHeadDim + hf * 8;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) qreg[cb][kb] = *reinterpret_cast<const u32x4*>(qp + kb * 16);
  }

  f32x16 o_acc[kCB][4];
  float m_run[kCB], l_part[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
#pragma unroll
    for (int db = 0; db < 4; ++db) o_acc[cb][db] = f32x16{};
    m_run[cb] = -INFINITY;
    l_part[cb] = 0.f;
  }

  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  // Staging assignment.  K: chunk (key tid/16 + 16 i, 16-byte column tid%16).
  // V: the four keys vkrow*4 .. +3 of 16-byte column vcol (8 dims); the
  // lane -> (vcol, vkrow) bit mapping makes the transposed LDS writes
  // conflict-free (see vt_offset).
  const int col = tid & 15;
  const int krow = tid >> 4;
  const int vcol = (lane & 7) | (((lane >> 4) & 1) << 3);
  const int vkrow = wave * 4 + (((lane >> 5) & 1) | (((lane >> 3) & 1) << 1));
  u32x4 kpre[4], vpre[4];

  auto prefetch = [&](int t) {
    const int k0 = t * kKT;
    const int64_t blk = table[k0 / kBlockSize];
    const int64_t base = ((blk * a.num_kv_heads + g) * kBlockSize + (k0 % kBlockSize)) * kHeadDim;
    const uint16_t* kt = a.k_cache + base + col * 8;
    const uint16_t* vt = a.v_cache + base + vcol * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      kpre[i] = *reinterpret_cast<const u32x4*>(kt + (krow + 16 * i) * kHeadDim);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vpre[i] = *reinterpret_cast<const u32x4*>(vt + (vkrow * 4 + i) * kHeadDim);
  };

  auto stage = [&](int t) {
    const int k0 = t * kKT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = krow + 16 * i;
      k_lds[key * 16 + (col ^ (key & 15))] = kpre[i];
    }
    // V rows past the context are zeroed: p = 0 there, and 0 * NaN poison
    // inside an MFMA would still be NaN.
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (k0 + vkrow * 4 + i >= n_k) vpre[i] = u32x4{0u, 0u, 0u, 0u};
    // transpose: dim d = vcol*8 + e receives keys vkrow*4 .. +3
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dims 2w (low halves) and 2w+1 (high halves) of the four keys
      const uint32_t lo01 = __builtin_amdgcn_perm(vpre[1][w], vpre[0][w], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(vpre[3][w], vpre[2][w], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(vpre[1][w], vpre[0][w], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(vpre[3][w], vpre[2][w], 0x07060302u);
      const int d0 = vcol * 8 + 2 * w;
      vt_lds[vt_offset(d0, vkrow)] = u32x2{lo01, lo23};
      vt_lds[vt_offset(d0 + 1, vkrow)] = u32x2{hi01, hi23};
    }
  };

  const float c = a.scale_log2;
  if (ntiles > 0) prefetch(0);
  for (int t = 0; t < ntiles; ++t) {
    if (t > 0) __syncthreads();
    stage(t);
    __syncthreads();
    if (t + 1 < ntiles) prefetch(t + 1);
    const int k0 = t * kKT;
    if (!wave_has_rows || k0 >= my_kend) continue;

    // ---- S^T = K Q^T for 2 x 32 keys and every column block ---------------
    f32x16 s_acc[kCB][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = kt * 32 + j;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const u32x4 av = k_lds[key * 16 + ((kb * 2 + hf) ^ (key & 15))];
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          s_acc[cb][kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(av), as_bf16x8(qreg[cb][kb]), kb == 0 ? f32x16{} : s_acc[cb][kt], 0, 0, 0);
      }
    }

    // ---- online softmax (base 2), one column block at a time --------------
    // element e = rr*4 + ee of s_acc[cb][kt] is key k0 + kt*32 + 8*rr + 4*hf + ee.
    const bool diag = (k0 + kKT - 1 > off + my_q0) || (k0 + kKT > n_k);
    u32x4 pfrag[kCB][4];  // B operands: (kt, ks) -> 16 keys
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      if (diag) {  // masked keys (past the query's position or the context) -> -inf
        const int lim = min(q_pos[cb], n_k - 1) - k0 - 4 * hf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int ko = kt * 32 + 8 * (e >> 2) + (e & 3);
            s_acc[cb][kt][e] = ko <= lim ? s_acc[cb][kt][e] : -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; e += 2)
          tmax = fmaxf(tmax, fmaxf(s_acc[cb][kt][e], s_acc[cb][kt][e + 1]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * c;  // both lane halves hold the query
      // Lazy rescaling: the running max only moves (and O, l are rescaled)
      // when a score exceeds it by more than kRescaleSlack (log2 units), so
      // p <= 2^kRescaleSlack stays well inside fp32/bf16 range.
      const bool grow = tmax > m_run[cb] + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? tmax : m_run[cb];
        const float alpha = grow ? fast_exp2(m_run[cb] - m_new) : 1.f;  // 0 when leaving -inf
        m_run[cb] = m_new;
        l_part[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o_acc[cb][db] *= alpha;
      }
      const float neg_m = m_run[cb] == -INFINITY ? 0.f : -m_run[cb];
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(s_acc[cb][kt][ks * 8 + e], c, neg_m));
          psum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
          pfrag[cb][kt * 2 + ks] = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                                         pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
        }
      l_part[cb] += psum;
    }

    // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + j;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // keys kt*32 + 16ks + 4hf + {0..3} and the same + 8, in one 16 bytes
          const u32x4 av = *reinterpret_cast<const u32x4*>(
              &vt_lds[vt_offset_chunk(d, kt * 4 + ks * 2 + hf)]);
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb)
            o_acc[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(av), as_bf16x8(pfrag[cb][kt * 2 + ks]), o_acc[cb][db], 0, 0, 0);
        }
    }
  }

  // ---- epilogue: out[q_row][h][d] = O^T[d][j] / l ---------------------------
  if (!wave_has_rows) return;
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const float l_tot = l_part[cb] + __shfl_xor(l_part[cb], 32, 64);
    if (qi[cb] >= n_q) continue;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    uint16_t* op = a.out + ((int64_t)(q_begin + qi[cb]) * a.num_q_heads + h) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = db * 32 + 8 * rr + 4 * hf;
        const u32x2 w =
            u32x2{pack_bf16(o_acc[cb][db][rr * 4] * inv, o_acc[cb][db][rr * 4 + 1] * inv),
                  pack_bf16(o_acc[cb][db][rr * 4 + 2] * inv, o_acc[cb][db][rr * 4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = w;
      }
  }
}

}  // namespace

bool prefill_supported_group(int group) { return group == 1 || group == 2 || group % 4 == 0; }

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
  a.heads_per_wg = a.group >= 4 ? 4 : a.group;
  a.pos_tiles = 4 / a.heads_per_wg;
  a.head_chunks = a.group / a.heads_per_wg;
  const int wg_rows = 32 * kWaveCB * a.pos_tiles;
  a.max_wg_tiles = (l.max_seqlen_q + wg_rows - 1) / wg_rows;
  a.scale_log2 = l.scale * kLog2e;
  a.out = (uint16_t*)l.out;
  const int64_t grid = (int64_t)a.max_wg_tiles * l.batch * l.num_kv_heads * a.head_chunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_kernel<kWaveCB>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
