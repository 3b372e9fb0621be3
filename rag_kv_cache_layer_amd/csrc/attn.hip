// Attention of the recomputed rows over the blended cache.
//
// CacheBlend (arXiv 2405.16444) section 4.2, Figure 5b: the K/V of the
// selected tokens are expanded with the reused entries of all other tokens, so
// that attention includes the selected tokens x all other tokens, and the
// same attention module produces the next layer's input.  Query row i (at
// cache row / position p_i) attends causally to cache rows 0 .. p_i; query
// head h reads KV head h / (n_q / n_kv).
//
// bf16 path (gfx950 matrix cores): one workgroup per (32 query rows, KV head,
// key split) with one wave per query head of the group, so the K/V tiles
// staged in LDS are shared by all heads that read them.  Each wave keeps its
// 32 queries' Q fragments in registers (two 16-column MFMA blocks, so every
// K or V fragment read from LDS feeds two MFMAs) and walks 64-key tiles with
// an online softmax in fp32 (base-2 exponent).  K and V tiles reach LDS by
// direct-to-LDS buffer loads into a ring of stages, the next tile's loads in
// flight while the current one is computed; rows past T read as zero.
// Scores are formed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16), so
// every lane owns one query column: the row statistics need only two
// cross-lane steps and the probabilities feed the P V product (O^T += V^T
// P^T) straight from registers -- the K index of an MFMA is a sum, so the
// same key permutation on both operands is exact.  V stays in its natural
// [key][dim] layout; its transposed operand comes from transposing LDS reads
// (ds_read_b64_tr_b16).  Both tiles' 16-byte chunks are XOR-swizzled per row
// so that these reads are free of bank conflicts.  The causal mask is applied
// only on tiles that reach past some row's position.  A key tile past a
// query's position is an exact no-op for it (alpha = 1, p = 0), so a row's
// result does not depend on the other rows of its tile.  Tiles holding the
// latest positions (the longest key ranges) go first.
//
// When there are too few (row tile, KV head) workgroups to fill the chip, the
// keys are split at fixed multiples of 512: each split writes an unnormalised
// partial (O rounded to bf16, which halves the partials' traffic; running max
// and sum in fp32) and a merge kernel combines a row's splits in fp32 in
// split order.  The split boundaries never depend on the other rows, so a row's
// result still does not either.
//
// fp32 path: one wave per (row, head); scores in LDS, two-pass softmax.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "cb_internal.h"

namespace cb {

namespace {

constexpr int kRowTile = kAttnRowTile;   // query rows per workgroup
#ifndef CB_ATTN_KT
#define CB_ATTN_KT 64
#endif
constexpr int kKeyTile = CB_ATTN_KT;   // keys per LDS stage (32 or 64)
static_assert(kKeyTile == 32 || kKeyTile == 64, "key tile");
#ifndef CB_ATTN_NS
#define CB_ATTN_NS 2
#endif
#ifndef CB_ATTN_MINB
#define CB_ATTN_MINB 2
#endif
// K/V tiles in the LDS ring: 2 (64 KB at head_dim 128) leaves room for two
// workgroups per CU, which measures faster than a deeper ring with one
constexpr int kStages = CB_ATTN_NS;
static_assert(kStages >= 2 && kStages <= 4, "ring depth");
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
// vector instructions placed between the matrix instructions of the two
// overlapped phases of a key tile (scores / mask-max, P V / probabilities)
#ifndef CB_ATTN_SG_B
#define CB_ATTN_SG_B 3
#endif
#ifndef CB_ATTN_SG_E
#define CB_ATTN_SG_E 4
#endif
// wave priority raised over the MFMA-dense parts of a tile (the scores, the
// P V products), so that the SIMD's other wave fills the matrix pipe's gaps
// with its vector work rather than competing for issue
// the first half's K fragment reads also all before its MFMAs
#ifndef CB_ATTN_FH
#define CB_ATTN_FH 1
#endif
#ifndef CB_ATTN_PRIO
#define CB_ATTN_PRIO 1
#endif
#define CB_PRIO(n)                                  \
  do {                                              \
    if constexpr (CB_ATTN_PRIO) __builtin_amdgcn_s_setprio(n); \
  } while (0)
// workgroups the key split aims at when the (row tile, KV head) grid is small
#ifndef CB_ATTN_WG_TARGET
#define CB_ATTN_WG_TARGET 768
#endif
#ifndef CB_ATTN_SPLIT
#define CB_ATTN_SPLIT 512
#endif
constexpr int kKeySplit = CB_ATTN_SPLIT;   // smallest key split (multiple of kKeyTile)
static_assert(kKeySplit % 64 == 0 && kKeySplit >= 512, "the partial buffers are sized for splits of >= 512 keys");

// Lazy rescale threshold of the online softmax, in base-2 units of the
// scores (0: the reference follows every new maximum)
#ifndef CB_ATTN_TAU
#define CB_ATTN_TAU 8
#endif
constexpr float kTau = CB_ATTN_TAU;

// Maximum / sum over the four lane groups that hold one query's keys (lanes
// q, q + 16, q + 32, q + 48) by the gfx950 row-swap permutes: after
// permlane16_swap(x, x) the two results hold the values of rows 0 / 1 (and
// 2 / 3) in every lane of those rows, after permlane32_swap those of the two
// halves, so combining the pair reduces over the partners (in the same order
// for every lane, up to the commutativity of the operation).
__device__ __forceinline__ float max4g(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}
__device__ __forceinline__ float sum4g(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

// One wave instruction: 16 bytes per lane from the buffer at byte offset
// `off` into LDS at lds + 16 * lane (loads past the buffer's end write zero).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}

// Rows, cache and length of a row tile.  With several requests each request's
// rows start a new tile, so a tile never mixes caches.
struct TileInfo {
  int r0, r1, T;
  const void* K;
  const void* V;
};

__device__ __forceinline__ TileInfo tile_info(const AttnArgs& a, int tile) {
  if (a.req.n == 0) return TileInfo{tile * kRowTile, min(a.m, tile * kRowTile + kRowTile), a.T, a.K, a.V};
  int r = 0;
  while (r + 1 < a.req.n && a.req.tile_off[r + 1] <= tile) ++r;
  const int r0 = a.req.row_off[r] + (tile - a.req.tile_off[r]) * kRowTile;
  return TileInfo{r0, min(a.req.row_off[r + 1], r0 + kRowTile), a.req.T[r], a.req.k[r], a.req.v[r]};
}

__device__ __forceinline__ int tile_of_row(const AttnArgs& a, int i) {
  if (a.req.n == 0) return i / kRowTile;
  const int r = req_of_row(a.req, i);
  return a.req.tile_off[r] + (i - a.req.row_off[r]) / kRowTile;
}

__host__ __device__ inline int n_row_tiles(const AttnArgs& a) {
  return a.req.n == 0 ? (a.m + kRowTile - 1) / kRowTile : a.req.tile_off[a.req.n];
}

template <int HD, int G>
__global__ __launch_bounds__(64 * G, G >= 2 ? CB_ATTN_MINB : 1) void attn_bf16_kernel(AttnArgs a, float scale_log2) {
  constexpr int KT = HD == 128 ? kKeyTile : 64;   // a head_dim-64 tile of 32 keys is too small for 8 waves
  constexpr int KB = KT / 16;                      // 16-key score blocks per tile
  constexpr int KS = KT / 32;                      // 32-key PV steps per tile
  constexpr int ROWB = HD * 2;                // bytes of one key row of a head
  constexpr int CPR = HD / 8;                 // 16-byte chunks per key row
  constexpr int RPB = 1024 / ROWB;            // key rows per 1 KB block
  constexpr int KPW = KT / RPB / G;           // blocks per tile that each wave loads
  constexpr int kTile = KT * ROWB;            // bytes of a K (or V) tile
  constexpr int kStage = 2 * kTile;
  constexpr int NS = (G == 1 && kStages > 3) ? 3 : kStages;   // DMA wait counts stay below 64
  static_assert(KPW >= 1 && KPW * RPB * G == KT, "tile rows must split evenly over the waves");
  __shared__ __attribute__((aligned(16))) char smem[NS * kStage];
  typedef __attribute__((address_space(1))) const u32x4_t gvec;
  // slot of 16-byte chunk c in key row r is c ^ fk(r) (K) or c ^ fv(r) (V):
  // K's fragment reads (16 rows, one chunk) and V's transposing reads (4
  // rows x 2 chunks per 16 lanes) then spread over all banks
  auto fk = [](int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto fv = [](int r) { return HD == 128 ? ((r & 3) << 1) | (((r >> 2) & 1) << 3) : ((r & 3) << 1); };

  // 1-D grid over (group = KV head + n_kv * key split, row tile).  Workgroups
  // are dealt round-robin to the 8 XCDs, each with its own L2; when the group
  // count is a multiple of 8, workgroup b runs group b % 8 + 8 j on XCD b % 8,
  // so every row tile that reads one group's K/V shares an L2 and the XCDs
  // get equal mixes of key splits.  Latest row tiles (longest key ranges)
  // come first within a group.
  const int n_tiles = n_row_tiles(a);
  const int n_groups = (int)gridDim.x / n_tiles;
  const int b = blockIdx.x;
  int grp, t;
  if ((n_groups & 7) == 0) {
    const int j = b >> 3;
    grp = (b & 7) + 8 * (j / n_tiles);
    t = j % n_tiles;
  } else {
    grp = b / n_tiles;
    t = b % n_tiles;
  }
  const int tile = n_tiles - 1 - t;
  const int kvh = grp % a.n_kv;
  const int split = grp / a.n_kv;
  const TileInfo ti = tile_info(a, tile);
  const int T_rows = ti.T;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int head = kvh * G + w;
  const int q = lane & 15, gp = lane >> 4;
  const int ldkv = a.n_kv * HD;
  // K/V of this KV head through buffer resources: rows at or past T lie
  // past the resource's end and load as zero (they are masked), and a
  // tile's row offset is a scalar operand
  const uint32_t row_bytes = (uint32_t)ldkv * 2;
  const uint32_t kv_span = (uint32_t)((int64_t)T_rows * ldkv * 2 - (int64_t)kvh * HD * 2);
  const __amdgpu_buffer_rsrc_t rK = make_rsrc((const bf16_t*)ti.K + kvh * HD, kv_span);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc((const bf16_t*)ti.V + kvh * HD, kv_span);

  // LDS ring of NS stages, each a K tile and a V tile of KT keys in their
  // natural [key][dim] layout, filled by direct-to-LDS loads: one wave
  // instruction fills a 1 KB block of RPB key rows; lane L fills 16-byte slot
  // L % CPR of row L / CPR with the dim chunk slot ^ f(row).
  uint32_t kof[KPW], vof[KPW];
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const int blk = w * KPW + j;   // 1 KB block of the tile
    const int row = blk * RPB + lane / CPR;
    const int slot = lane % CPR;
    kof[j] = (uint32_t)row * row_bytes + (uint32_t)((slot ^ fk(row)) << 4);
    vof[j] = (uint32_t)row * row_bytes + (uint32_t)((slot ^ fv(row)) << 4);
  }
  auto issue = [&](int stage, int t0) {
    char* sk = smem + stage * kStage;
    char* sv = sk + kTile;
    const uint32_t so = (uint32_t)t0 * row_bytes;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int blk = w * KPW + j;
      dma16(rK, sk + blk * 1024, kof[j] + so);
      dma16(rV, sv + blk * 1024, vof[j] + so);
    }
  };

  // Q fragments of both 16-row blocks go out first (their addresses need no
  // position), then the rows' positions and the first key tiles: the
  // workgroup waits once for all of it
  bool valid[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) valid[b] = ti.r0 + b * 16 + q < ti.r1;
  const int ldq = a.n_q * HD;
  bf16x8_t qf[2][HD / 32];
  auto load_q = [&](const int (&qr)[2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const gvec* Qp = (const gvec*)((const bf16_t*)a.Q + (int64_t)qr[b] * ldq + head * HD + gp * 8);
#pragma unroll
      for (int ks = 0; ks < HD / 32; ++ks) {
        u32x4_t u = valid[b] ? Qp[ks * 4] : u32x4_t{0u, 0u, 0u, 0u};
        qf[b][ks] = __builtin_bit_cast(bf16x8_t, u);
      }
    }
  };
  // (two uniform paths, so that the common one, Q rows in row order, waits
  // for no index load before issuing the fragment loads)
  if (a.qmap) {
    int qr[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) qr[b] = valid[b] ? a.qmap[ti.r0 + b * 16 + q] : 0;
    load_q(qr);
  } else {
    int qr[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) qr[b] = valid[b] ? ti.r0 + b * 16 + q : 0;
    load_q(qr);
  }
  int praw[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int i = ti.r0 + b * 16 + q;
    praw[b] = valid[b] ? (a.qpos ? a.qpos[i] : i) : 0;
  }
  // the first NS-1 key tiles of the split go out while the Q fragments and
  // positions are in flight: their start k_lo does not depend on the
  // positions (tiles past the key range are never read; a workgroup with no
  // keys waits for them before it ends)
  const int k_lo = a.key_split > 0 ? split * a.key_split : 0;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st, k_lo + st * KT);
  int pos[2];
  int pm = 0, pmin = INT_MAX;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int p = praw[b];
    pos[b] = p < 0 ? 0 : (p >= T_rows ? T_rows - 1 : p);
    pm = max(pm, pos[b]);
    if (valid[b]) pmin = min(pmin, pos[b]);
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    pm = max(pm, __shfl_xor(pm, o));
    pmin = min(pmin, __shfl_xor(pmin, o));
  }
  // key range of this workgroup
  const bool splitting = a.key_split > 0 && pm >= a.key_split;
  const int k_hi = splitting ? min(pm + 1, k_lo + a.key_split) : pm + 1;
  if (k_lo >= k_hi) {   // uniform over the workgroup
    CB_WAIT_VMCNT(0);
    return;
  }

  f32x4_t oacc[2][HD / 16];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int mb = 0; mb < HD / 16; ++mb) oacc[b][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const int n_it = (k_hi - k_lo + KT - 1) / KT;
  // V^T operand reads: lane L = 16 g + 4 j + c4 points at the 4 dims
  // 16 mb + 4 c4 .. +3 of key 32 st + 4 g + j (+ 16 for the second read);
  // the transposing read hands lane 16 g + i the values of dim 16 mb + i for
  // the 4 keys, i.e. k slots 8 g .. 8 g + 7 of the MFMA's A operand
  const int tj = (lane >> 2) & 3, tc = lane & 3;
  const int tkey = 4 * gp + tj;                           // + 32 st (+ 16)

  for (int it0 = 0; it0 < n_it; it0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int it = it0 + u;
      if (it >= n_it) break;
      const int t0 = k_lo + it * KT;
      // this wave's loads of tile `it` landed once at most the later tiles'
      // loads are outstanding; then every wave's have (barrier)
      const int later = min(n_it - 1 - it, NS - 2);
      if (later >= 2) CB_WAIT_VMCNT(4 * KPW);
      else if (later == 1) CB_WAIT_VMCNT(2 * KPW);
      else CB_WAIT_VMCNT(0);
      CB_BARRIER();
      if (it + NS - 1 < n_it) issue((u + NS - 1) % NS, t0 + (NS - 1) * KT);
      const char* sk = smem + u * kStage;
      const char* sv = sk + kTile;

      // S^T[key][query]: lane holds keys t0+16kb+4gp+v of queries q (b=0) and 16+q (b=1).
      // The tile is worked in two halves of 32 keys with an explicit
      // instruction schedule, so that the matrix cores run one half while the
      // vector units work on the other: the second half's scores are formed
      // while the first half is masked and reduced, and the first half's
      // P V product runs while the second half's probabilities are formed.
      // The arithmetic per query and its order are those of one 64-key pass.
      auto tile_body = [&](auto masked_c) {
        constexpr bool MASKED = decltype(masked_c)::value;
        f32x4_t s[2][KB];
        auto scores = [&](int kb) {
          s[0][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          s[1][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          const int key = kb * 16 + q;
#pragma unroll
          for (int ks = 0; ks < HD / 32; ++ks) {
            const int c = ks * 4 + gp;
            const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(sk + key * ROWB + ((c ^ fk(key)) << 4));
            s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], s[0][kb], 0, 0, 0);
            s[1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][ks], s[1][kb], 0, 0, 0);
          }
        };
        float mx[2] = {-INFINITY, -INFINITY};
        auto mask_max = [&](int kb) {
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              if constexpr (MASKED) {
                const int key = t0 + kb * 16 + 4 * gp + v;
                s[b][kb][v] = key <= pos[b] ? s[b][kb][v] : -INFINITY;
              }
              mx[b] = fmaxf(mx[b], s[b][kb][v]);
            }
        };
        CB_PRIO(1);
#pragma unroll
        for (int kb = 0; kb < KB / 2; ++kb) scores(kb);
#if CB_ATTN_FH
        __builtin_amdgcn_sched_group_barrier(0x100, (KB / 2) * (HD / 32), 0);   // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, KB * (HD / 32), 0);         // MFMA
#endif
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = KB / 2; kb < KB; ++kb) scores(kb);
#pragma unroll
        for (int kb = 0; kb < KB / 2; ++kb) mask_max(kb);
        // second half's scores (K fragment reads + MFMAs) interleaved with the
        // first half's mask and max
        // (all of the half's K fragment reads go first, so that each MFMA pair
        // waits only for its own fragment, not for a read issued just before)
        constexpr int NB = (KB / 2) * (HD / 32);   // K fragment reads, one per MFMA pair
        __builtin_amdgcn_sched_group_barrier(0x100, NB, 0);   // LDS reads
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, CB_ATTN_SG_B, 0);   // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = KB / 2; kb < KB; ++kb) mask_max(kb);
        CB_PRIO(0);
        // online softmax per query, in base-2 units (x = s * scale_log2, one
        // fused multiply-add inside the exponent).  The reference maximum
        // m_run moves only when the tile's maximum exceeds it by more than
        // kTau (the exponents then stay below 2^kTau); the output and the sum
        // are relative to the same reference, so the result is the softmax
        // up to rounding, and a row's arithmetic depends on its own scores only
        bf16x8_t pb[2][KS];
        float alpha[2], m_use[2], sum[2] = {0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const float mt = max4g(mx[b]) * scale_log2;
          const bool grow = mt > m_run[b] + kTau;   // also the first keys of a row (m_run = -inf)
          alpha[b] = grow ? __builtin_amdgcn_exp2f(m_run[b] - mt) : 1.f;
          m_run[b] = grow ? mt : m_run[b];
          m_use[b] = m_run[b] == -INFINITY ? 0.f : m_run[b];   // a fully masked row stays empty
        }
        // the output accumulators are rescaled only when some row's reference
        // moved (a multiplication by exactly 1 for the others)
        if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.f || alpha[1] != 1.f) != 0) {
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int mb = 0; mb < HD / 16; ++mb) oacc[b][mb] *= alpha[b];
        }
        // probabilities of the 32-key step st; P^T as the B operand: k slot j
        // of lane group gp is key 32st+4gp+j (j<4) or 32st+16+4gp+(j-4),
        // matching the V^T reads below
        auto probs = [&](int st) {
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const float e =
                    __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][2 * st + h][v], scale_log2, -m_use[b]));
                sum[b] += e;
                pb[b][st][4 * h + v] = (__bf16)e;
              }
        };
        // the output accumulators are rescaled by alpha (exactly 1 when the
        // running max did not grow) right before the P V product adds to them
        auto pv = [&](int st) {
#pragma unroll
          for (int mb = 0; mb < HD / 16; ++mb) {
            const int c = 2 * mb + (tc >> 1), h8 = (tc & 1) * 8;
            const int k1 = 32 * st + tkey, k2 = k1 + 16;
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s*)(sv + k1 * ROWB + ((c ^ fv(k1)) << 4) + h8));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s*)(sv + k2 * ROWB + ((c ^ fv(k2)) << 4) + h8));
            const bf16x8_t va =
                __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[0][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[0][st], oacc[0][mb], 0, 0, 0);
            oacc[1][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[1][st], oacc[1][mb], 0, 0, 0);
          }
        };
        probs(0);
        __builtin_amdgcn_sched_barrier(0);
        CB_PRIO(1);
        pv(0);
        probs(1);
        // first half's P V (transposing LDS reads + MFMAs, rescale) interleaved
        // with the second half's probabilities
        // (all transposing reads of the half first, as for the scores)
        constexpr int NP = HD / 16;   // V^T fragment read pairs, one per MFMA pair
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * NP, 0);   // LDS reads
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, CB_ATTN_SG_E, 0);   // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        pv(1);
        CB_PRIO(0);
#pragma unroll
        for (int b = 0; b < 2; ++b) l_run[b] = l_run[b] * alpha[b] + sum4g(sum[b]);
      };
      // causal mask only on tiles that reach past some row's position
      // (uniform: every wave of the workgroup has the same rows)
      if (t0 + KT - 1 > pmin) tile_body(std::true_type{});
      else tile_body(std::false_type{});
    }
  }
  CB_WAIT_VMCNT(0);
  if (a.fin_ids_out && kvh == 0 && split == 0 && w == 0) {
    // selection outputs of a layer that keeps every row (one wave per row
    // tile, after its own attention work: nothing in the kernel reads them)
    for (int i = ti.r0 + lane; i < ti.r1; i += 64) {
      a.fin_ids_out[i] = a.fin_ids_in[i];
      float sdev;
      if (i < a.fin_n_cand) {
        sdev = 0.f;
        for (int t = 0; t < a.fin_n_parts; ++t) sdev += a.fin_dev_part[(int64_t)t * a.fin_ld_part + i];
      } else {
        sdev = __builtin_nanf("");
      }
      a.fin_dev[i] = sdev;
    }
  }

#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (!valid[b]) continue;
    const int i = ti.r0 + b * 16 + q;
    if (!splitting) {
      bf16_t* Op = (bf16_t*)a.O + (int64_t)i * ldq + head * HD + 4 * gp;
#pragma unroll
      for (int mb = 0; mb < HD / 16; ++mb) {
        float o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = oacc[b][mb][v] / l_run[b];
        const uint32_t w0 = (uint32_t)f2bf(o[0]) | ((uint32_t)f2bf(o[1]) << 16);
        const uint32_t w1 = (uint32_t)f2bf(o[2]) | ((uint32_t)f2bf(o[3]) << 16);
        *reinterpret_cast<uint2*>(Op + mb * 16) = make_uint2(w0, w1);
      }
    } else {
      // unnormalised partial of this key split, merged by attn_merge_kernel
      const int64_t slot = ((int64_t)split * a.m + i) * a.n_q + head;
      bf16_t* Op = a.o_part + slot * HD + 4 * gp;
#pragma unroll
      for (int mb = 0; mb < HD / 16; ++mb) {
        const uint32_t w0 = (uint32_t)f2bf(oacc[b][mb][0]) | ((uint32_t)f2bf(oacc[b][mb][1]) << 16);
        const uint32_t w1 = (uint32_t)f2bf(oacc[b][mb][2]) | ((uint32_t)f2bf(oacc[b][mb][3]) << 16);
        *reinterpret_cast<uint2*>(Op + mb * 16) = make_uint2(w0, w1);
      }
      if (gp == 0) *reinterpret_cast<float2*>(a.ml_part + slot * 2) = make_float2(m_run[b], l_run[b]);
    }
  }
}

// Merge the key-split partials of one row in split order, for every head:
// out = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s over the splits that
// hold keys of the row.  Rows of tiles that were not split are skipped.  One
// workgroup per (row, group of heads); HD / 4 threads per head, 4 dims each.
// Every thread reads its head's (max, sum) pairs itself and issues its loads
// before the workgroup learns whether the row's tile was split, so the
// kernel is about two memory round trips deep (the partial buffers are
// always in bounds; values read for a tile that was not split are dropped).
template <int HD>
constexpr int merge_heads() { return 256 / (HD / 4); }

// four consecutive bf16 partial values as fp32
__device__ __forceinline__ float4 ld_bf16x4(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
constexpr int kMergeRegs = 8;   // splits a merge thread holds in registers at once

template <int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  __shared__ int s_pm;
  constexpr int kTPH = HD / 4;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int head = blockIdx.y * merge_heads<HD>() + tid / kTPH;
  const int c = (tid % kTPH) * 4;
  // the attention workgroup of this row's tile decided whether to split
  const TileInfo ti = tile_info(a, tile_of_row(a, i));
  if (tid < 64) {
    const int r = ti.r0 + tid;
    int p = 0;
    if (tid < kRowTile && r < ti.r1) {
      p = a.qpos ? a.qpos[r] : r;
      p = p < 0 ? 0 : (p >= ti.T ? ti.T - 1 : p);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) p = max(p, __shfl_xor(p, o));
    if (tid == 0) s_pm = p;
  }
  int p = a.qpos ? a.qpos[i] : i;
  p = p < 0 ? 0 : (p >= ti.T ? ti.T - 1 : p);
  const int ns = p / a.key_split + 1;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  if (head < a.n_q) {
    const int64_t stride = (int64_t)a.m * a.n_q;   // slots per split
    const int64_t slot0 = (int64_t)i * a.n_q + head;
    if (ns <= kMergeRegs) {
      // every split's (max, sum) and output slice loaded at once (one memory
      // round trip), then the same arithmetic in the same order as below
      float2 ml[kMergeRegs];
      float4 o[kMergeRegs];
#pragma unroll
      for (int sp = 0; sp < kMergeRegs; ++sp) {
        if (sp < ns) {
          const int64_t slot = slot0 + sp * stride;
          ml[sp] = *reinterpret_cast<const float2*>(a.ml_part + slot * 2);
          o[sp] = ld_bf16x4(a.o_part + slot * HD + c);
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sp = 0; sp < kMergeRegs; ++sp)
        if (sp < ns) mx = fmaxf(mx, ml[sp].x);
#pragma unroll
      for (int sp = 0; sp < kMergeRegs; ++sp) {
        if (sp < ns) {
          const float wgt = exp2f(ml[sp].x - mx);
          den += wgt * ml[sp].y;
          num.x += wgt * o[sp].x; num.y += wgt * o[sp].y; num.z += wgt * o[sp].z; num.w += wgt * o[sp].w;
        }
      }
    } else {
      float mx = -INFINITY;
#pragma unroll 8
      for (int sp = 0; sp < ns; ++sp) mx = fmaxf(mx, a.ml_part[(slot0 + sp * stride) * 2]);
#pragma unroll 8
      for (int sp = 0; sp < ns; ++sp) {
        const int64_t slot = slot0 + sp * stride;
        const float2 ml = *reinterpret_cast<const float2*>(a.ml_part + slot * 2);
        const float4 o = ld_bf16x4(a.o_part + slot * HD + c);
        const float wgt = exp2f(ml.x - mx);
        den += wgt * ml.y;
        num.x += wgt * o.x; num.y += wgt * o.y; num.z += wgt * o.z; num.w += wgt * o.w;
      }
    }
  }
  __syncthreads();
  if (s_pm < a.key_split || head >= a.n_q) return;   // tile written directly
  const float inv = 1.0f / den;
  bf16_t* Op = (bf16_t*)a.O + ((int64_t)i * a.n_q + head) * HD + c;
  const uint32_t w0 = (uint32_t)f2bf(num.x * inv) | ((uint32_t)f2bf(num.y * inv) << 16);
  const uint32_t w1 = (uint32_t)f2bf(num.z * inv) | ((uint32_t)f2bf(num.w * inv) << 16);
  *reinterpret_cast<uint2*>(Op) = make_uint2(w0, w1);
}

__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a, float scale) {
  extern __shared__ float sc[];
  __shared__ float qs[256];
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int hd = a.hd;
  const int kvh = h / (a.n_q / a.n_kv);
  const void* K = a.K;
  const void* V = a.V;
  int T_rows = a.T;
  if (a.req.n > 0) {
    const int r = req_of_row(a.req, i);
    K = a.req.k[r];
    V = a.req.v[r];
    T_rows = a.req.T[r];
  }
  int p = a.qpos ? a.qpos[i] : i;
  p = p < 0 ? 0 : (p >= T_rows ? T_rows - 1 : p);
  const int qr = a.qmap ? a.qmap[i] : i;
  const float* Qp = (const float*)a.Q + (int64_t)qr * a.n_q * hd + h * hd;
  for (int d = lane; d < hd; d += 64) qs[d] = Qp[d];
  __syncthreads();
  const int ldkv = a.n_kv * hd;
  const float* Kg = (const float*)K + kvh * hd;
  const float* Vg = (const float*)V + kvh * hd;
  float mx = -INFINITY;
  for (int t = lane; t <= p; t += 64) {
    const float* kr = Kg + (int64_t)t * ldkv;
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s += qs[d] * kr[d];
    s *= scale;
    sc[t] = s;
    mx = fmaxf(mx, s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float sum = 0.f;
  for (int t = lane; t <= p; t += 64) {
    const float e = expf(sc[t] - mx);
    sc[t] = e;
    sum += e;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  __syncthreads();
  float* Op = (float*)a.O + (int64_t)i * a.n_q * hd + h * hd;
  for (int d = lane; d < hd; d += 64) {
    float acc = 0.f;
    for (int t = 0; t <= p; ++t) acc += sc[t] * Vg[(int64_t)t * ldkv + d];
    Op[d] = acc / sum;
  }
}

template <int HD>
hipError_t launch_bf16_hd(const AttnArgs& a, hipStream_t s, float scale_log2) {
  const int g = a.n_q / a.n_kv;
  const int n_split = a.key_split > 0 ? (a.T + a.key_split - 1) / a.key_split : 1;
  const dim3 grid(n_row_tiles(a) * a.n_kv * n_split);
  {
    LaunchScope ls("attention", s);
    switch (g) {
      case 1: attn_bf16_kernel<HD, 1><<<grid, 64, 0, s>>>(a, scale_log2); break;
      case 2: attn_bf16_kernel<HD, 2><<<grid, 128, 0, s>>>(a, scale_log2); break;
      case 4: attn_bf16_kernel<HD, 4><<<grid, 256, 0, s>>>(a, scale_log2); break;
      case 8: attn_bf16_kernel<HD, 8><<<grid, 512, 0, s>>>(a, scale_log2); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.key_split <= 0) return e;
  LaunchScope ls("attn_merge", s);
  constexpr int hpb = merge_heads<HD>();
  attn_merge_kernel<HD><<<dim3(a.m, (a.n_q + hpb - 1) / hpb), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int attn_key_split(int dtype, int m, int n_kv, int T) {
  if (dtype != CB_BF16) return 0;
  const int groups = (m + kRowTile - 1) / kRowTile * n_kv;
  if (groups >= 512) return 0;
  // about 1.5 workgroups per slot (two per CU): the keys in ~768 / groups
  // parts, each a whole number of key tiles and at least kKeySplit keys (the
  // partial buffers hold T / kKeySplit splits).  At the 8B layer (128
  // groups, T = 3104) that is 6 parts of 576 keys: attention + merge 47 us,
  // against 55 us with 7 parts of 512 and 52 us with 4 of 832.
  const int parts = std::max(1, (CB_ATTN_WG_TARGET + groups / 2) / groups);
  const int per = (T + parts - 1) / parts;
  return std::max(kKeySplit, (per + 63) / 64 * 64);
}

size_t attn_part_rows(int n_q, int n_kv) {
  (void)n_q;
  return (size_t)kRowTile * ((512 + n_kv - 1) / n_kv);
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s) {
  if (a.m <= 0) return hipSuccess;
  if (dtype == CB_BF16) {
    const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)a.hd));
    if (a.hd == 128) return launch_bf16_hd<128>(a, s, scale_log2);
    if (a.hd == 64) return launch_bf16_hd<64>(a, s, scale_log2);
    return hipErrorInvalidValue;
  }
  const float scale = (float)(1.0 / __builtin_sqrt((double)a.hd));
  LaunchScope ls("attention", s);
  attn_f32_kernel<<<dim3(a.m, a.n_q), 64, (size_t)a.T * sizeof(float), s>>>(a, scale);
  return hipGetLastError();
}

}  // namespace cb
