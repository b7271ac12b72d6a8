// Internal: the chunked-prefill attention work item, shared by the prefill
// kernel and the mixed-batch kernel.
//
// Prefill runs the prompt in parallel and is mostly matrix-matrix work
// (aiwithghost.com "KV cache and continuous batching: 1,000 people ask AI",
// section "What does a KV cache keep?"); it is capped at a fixed token budget
// per step so decode waits at most one chunk (gouthm.com "The KV cache is not
// your bottleneck", section "The fix that mattered"), and it can start after a
// prefix whose K/V are already cached (daviddominguez.dev "The KV cache and
// prefix caching", section "A prefix already in the cache can skip its
// prefill"). This is the one dense contraction of the path, so it runs on MFMA.
//
// Tiling (one work item = 8 waves = 256 query rows of one kv head):
//   row r <-> (position qt*MP + r / G, query head kvh*G + r % G), MP = 256 / G,
//   so the G query heads that share a K/V head share every K/V tile.
//   Keys are walked in tiles of 64 (four 16-token blocks through the block
//   table). Per tile and wave (2 row tiles of 16):
//     S^T[key][row] = K . Q^T          MFMA, A = K from LDS, B = Q from registers
//     online softmax per row            each lane owns one row (lane % 16)
//     O^T[dim][row] += V^T . P^T       MFMA, A = V^T from LDS, B = P from the S^T
//                                       registers (no transpose of P needed)
//   bf16: v_mfma_f32_16x16x32_bf16 (V staged transposed in LDS);
//   fp32: v_mfma_f32_16x16x4_f32 (V read row-major, one element per lane).
//   The reduction order inside an MFMA over keys is a permutation of the keys
//   (key 16m + 4g + i for lane group g); A and B use the same permutation.
//   The three steps are software-pipelined across key tiles so that the
//   softmax of one tile overlaps the PV product of the previous one.

#pragma once

#include <math.h>

#include <type_traits>

#include "kvc.h"
#include "kvc_append.h"
#include "kvc_device.h"

namespace kvc {

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kRowTiles = 2;                        // 16-row tiles per wave
constexpr int kRows = kPfWaves * kRowTiles * 16;    // 256 query rows per workgroup
constexpr int kKeyTile = 64;                        // keys per staged tile
constexpr int kWaitVmcnt0 = 0x0F70;                 // s_waitcnt vmcnt(0) (expcnt, lgkmcnt: no wait)
constexpr uint32_t kBf16OnePair = 0x3F803F80u;      // bf16 (1, 1)
constexpr uint32_t kDmaPastEnd = 0x7FFFFFF0u;        // buffer offset past any range: the load writes zeros

typedef __attribute__((address_space(3))) void lds_void;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Over each group of 16
// lanes, lane i addresses 4 consecutive 16-bit elements A_i; lane j receives
// A_{4k + j/4}[j % 4] for k = 0..3. The compiler counts these reads with the
// other LDS reads, so its waits for K and V fragments are exact. Without alias
// information on the read it would also wait for every buffer->LDS load in
// flight (draining the tile prefetch); the restrict parameter gives the
// inlined read a scope of its own, as the plain K-fragment loads have. The
// tile loads are ordered by the explicit waits and barriers that publish each
// tile.
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
__device__ __forceinline__ u32x2 tr_read_at(lds_s16x4* __restrict__ p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
}
template <int OFF>
__device__ __forceinline__ u32x2 tr_read_b64(uint32_t lds_addr) {
  return tr_read_at(reinterpret_cast<lds_s16x4*>((uintptr_t)(lds_addr + OFF)));
}

template <typename T> struct PfMfma;
template <> struct PfMfma<bf16_tag> {
  static constexpr int K = 32;                      // reduction depth per instruction
  using Frag = bf16x8_t;
  __device__ static f32x4 mma(const Frag& a, const Frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct PfMfma<float> {
  static constexpr int K = 4;
  using Frag = float;
  __device__ static f32x4 mma(const Frag& a, const Frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Softmax weights of one key tile as the PV product consumes them: bf16 pairs
// packed as MFMA B fragments, or fp32 one per (key tile, row tile, element).
template <bool BF16> struct PfP;
template <> struct PfP<true> { struct Tile { u32x4 v[2][kRowTiles]; }; };
template <> struct PfP<false> { struct Tile { float v[4][kRowTiles][4]; }; };

// Type the prefill computes in: fp8 tiles are dequantised to bf16 in LDS.
template <typename T>
using PfComputeT = std::conditional_t<std::is_same_v<T, fp8_tag>, bf16_tag, T>;

template <typename T, int D, int G>
struct PfShape {
  static constexpr int EB = ElemBytes<T>::value;
  static constexpr int RB = D * EB;                 // bytes per K row in LDS
  static constexpr int NC = RB / 16;                // 16-byte chunks per row
  static constexpr int MP = kRows / G;              // positions per workgroup
  static constexpr int KS = D / PfMfma<T>::K;       // k-steps over head_dim
  static constexpr int DT = D / 16;                 // output dim tiles
  static constexpr bool BF16 = (EB == 2);
  static constexpr int VT_STRIDE = kKeyTile + 8;    // padded V^T row (elements), bf16 only
  static constexpr int K_UNITS = kKeyTile * NC;     // 16-byte chunks of a K tile
  static constexpr int KPT = (K_UNITS + kPfThreads - 1) / kPfThreads;
  // V staging units: bf16 = (key pair, chunk) transposed on the way in; fp32 = chunk
  static constexpr int V_UNITS = BF16 ? (kKeyTile / 2) * NC : K_UNITS;
  static constexpr int VPT = (V_UNITS + kPfThreads - 1) / kPfThreads;
  static constexpr int VCH = BF16 ? 2 : 1;          // chunks per V unit
  static constexpr int K_LDS = kKeyTile * RB;
  static constexpr int V_LDS = BF16 ? D * VT_STRIDE * 2 : kKeyTile * RB;
  // tiles of 64 and 128 bf16 dims (bf16 or fp8 caches) go into NBUF K and
  // NBUF V buffers, both row-major with a chunk swizzle (bf16 by buffer->LDS
  // loads, fp8 through registers); the others go through registers into two K
  // and two (transposed) V buffers
  static constexpr bool DMA_OK = BF16 && NC >= 8;
  static constexpr int NBUF = 4;
  static constexpr int BPB = 16 * RB / 1024;        // 1 KB staging loads per 16-token block
  static constexpr int TILES_REG = 2 * K_LDS + 2 * V_LDS;
  static constexpr int TILES_DMA = DMA_OK ? 2 * NBUF * K_LDS : 0;
  static constexpr int TILES = TILES_REG > TILES_DMA ? TILES_REG : TILES_DMA;
  // pool rows of the blocks a workgroup reads, kept in LDS: 8,192 blocks
  // (131,072 keys) where the tile buffers leave room, else 2,048
  static constexpr int BT_CACHE = TILES <= 96 * 1024 ? 8192 : 2048;
  static constexpr int SMEM = TILES + BT_CACHE * 4;
  static_assert(kRows % G == 0, "G divides the row count");
};

struct PrefillArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* cu;
  const int32_t* prefix;
  const int32_t* bt;
  void* out;
  int32_t* err;
  int32_t hkv;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t total;
  int32_t max_chunk;
  int32_t n_qt;       // query tiles per sequence (grid decomposition)
  int32_t n_split;    // key-range splits per query tile (1: no split, rows written directly)
  int32_t split_tiles;  // key tiles per split
  int32_t n_work;     // n_qt * n_split * hkv * n_seqs
  int32_t n_cus;      // compute units and XCDs of the device (the workgroup deal)
  int32_t n_xcd;
  float scale_log2;
  float* ws_o;        // split partials: [total][Hq][n_split][D] fp32, unnormalised
  float2* ws_ml;      // [total][Hq][n_split] (running max in log2 units, row sum)
  const float* ks;    // fp8 caches: row scales [num_blocks][hkv][16] of K and V
  const float* vs;
};

constexpr int kMaxRankedSeqs = 64;    // one per lane of a wave

// The sequence whose prefill cost (chunk length x mean keys per query) has rank
// `rank` among the first n_seqs <= 64 (0 = costliest, ties by index). Every
// wave computes it alone: lane i counts the sequences costlier than i.
__device__ __forceinline__ int seq_with_cost_rank(const PrefillArgs& a, int n_seqs, int rank) {
  const int lane = threadIdx.x & 63;
  int64_t cost = -1;
  if (lane < n_seqs) {
    const int64_t c = a.cu[lane + 1] - a.cu[lane];
    cost = c * (2 * (int64_t)a.prefix[lane] + c);
  }
  const int lo = (int)(uint32_t)cost, hi = (int)(cost >> 32);
  int mine = 0;
  for (int m = 0; m < n_seqs; ++m) {
    const int64_t cm = (int64_t)(((uint64_t)(uint32_t)__shfl(hi, m, 64) << 32) | (uint32_t)__shfl(lo, m, 64));
    mine += (cm > cost || (cm == cost && m < lane)) ? 1 : 0;
  }
  const uint64_t hit = __ballot(lane < n_seqs && mine == rank);   // exactly one lane
  return __builtin_ctzll(hit);
}

template <typename T>
__device__ __forceinline__ void store4(void* out, size_t idx, const f32x4& v, float inv);
template <>
__device__ __forceinline__ void store4<float>(void* out, size_t idx, const f32x4& v, float inv) {
  *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx) =
      f32x4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
}
template <>
__device__ __forceinline__ void store4<bf16_tag>(void* out, size_t idx, const f32x4& v, float inv) {
  *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + idx) =
      u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
}

// One work item: query tile qt, key range sp, kv head kvh of sequence s (work
// = qt + n_qt * (sp + n_split * (kvh + hkv * s))), run by the 8 waves of the
// calling workgroup; every thread calls it (tid = its thread index), smem
// holds PfShape<T, D, G>::SMEM bytes. The chunk's K/V must already be in the
// cache.
template <typename T, int D, int G>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, int work, uint8_t* smem,
                                             int tid = threadIdx.x) {
  // fp8 caches are dequantised to bf16 as their tiles are staged into LDS
  // (code * row scale, rounded to bf16) and then take the bf16 path
  constexpr bool F8 = std::is_same_v<T, fp8_tag>;
  using CT = PfComputeT<T>;
  using S = PfShape<CT, D, G>;
  using M = PfMfma<CT>;
  using Frag = typename M::Frag;
  constexpr int RB_MEM = F8 ? D : S::RB;              // bytes of one cached row
  // bf16 and fp8 caches of 64 / 128 dims run the two-group pipeline over
  // row-major swizzled tiles; bf16 tiles go from the pool straight into LDS
  // (buffer->LDS loads), fp8 tiles through registers, converted on the way
  constexpr bool TWO = S::DMA_OK;
  constexpr bool DMA = TWO && !F8;
  int32_t* bt_lds = reinterpret_cast<int32_t*>(smem + S::TILES);
  const int qt = work % a.n_qt;
  const int sp = (work / a.n_qt) % a.n_split;
  const int kvh = (work / (a.n_qt * a.n_split)) % a.hkv;
  const int s = work / (a.n_qt * a.n_split * a.hkv);
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int t0 = a.cu[s];
  const int C = a.cu[s + 1] - t0;
  const int p0 = a.prefix[s];
  const int pos_lo = qt * S::MP;
  if (!chunk_ok(t0, C, p0, a.total, a.max_chunk)) {
    if (qt == 0 && sp == 0 && kvh == 0 && tid == 0) flag_error(a.err, KVC_DEVERR_CONTEXT);
    return;
  }
  if (pos_lo >= C) return;
  const int kv_len = p0 + C;                           // keys that exist after the write
  const int last_pos = p0 + min(pos_lo + S::MP, C) - 1;
  const int hq_all = a.hkv * G;
  // this workgroup's key tiles: [t_begin, t_end) of the ones its rows reach
  const int t_begin = sp * a.split_tiles;
  const int t_end = min(last_pos / kKeyTile + 1, t_begin + a.split_tiles);
  if (sp == a.n_split - 1 && last_pos / kKeyTile + 1 > t_begin + a.split_tiles && tid == 0)
    flag_error(a.err, KVC_DEVERR_CONTEXT);             // keys past max_context_len

  if (t_begin >= t_end) {
    // a split past this query tile's keys: an empty partial for each of its rows
    const int rows = min(S::MP, C - pos_lo) * G;
    for (int r = tid; r < rows; r += kPfThreads) {
      const size_t pr = ((size_t)(t0 + pos_lo + r / G) * hq_all + kvh * G + r % G) * a.n_split + sp;
      a.ws_ml[pr] = float2{-INFINITY, 0.f};
      for (int d = 0; d < D; d += 4)
        *reinterpret_cast<f32x4*>(a.ws_o + pr * D + d) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;

  // The pool row (block id * Hkv + kv head) of every block this workgroup
  // reads, validated once and cached in LDS; -1 for a block that holds no key
  // or has an id outside the pool. Contract violations are collected per lane
  // and flagged once at the end.
  const int nb_need = (min(kv_len, t_end * kKeyTile) + 15) / 16;
  int bad = 0;
  auto pool_row = [&](int lb) -> int {
    if (lb >= nb_need) return -1;
    if (lb >= a.max_blocks) {
      bad |= KVC_DEVERR_CONTEXT;
      return -1;
    }
    const int blk = bt_row[lb];
    if ((unsigned)blk >= (unsigned)a.num_blocks) {
      bad |= KVC_DEVERR_BLOCK_ID;
      return -1;
    }
    return blk * a.hkv + kvh;
  };
  const int lb0 = 4 * t_begin;                         // cache entry 0 = block lb0
  for (int i = tid; i < min(4 * (t_end - t_begin + 1), S::BT_CACHE); i += kPfThreads)
    bt_lds[i] = pool_row(lb0 + i);

  // rows owned by this lane: r = w*32 + n*16 + l16
  int row_pos[kRowTiles];                              // absolute position (clamped)
  bool row_ok[kRowTiles];
  Frag qf[kRowTiles][S::KS];
#pragma unroll
  for (int n = 0; n < kRowTiles; ++n) {
    const int r = w * (kRowTiles * 16) + n * 16 + l16;
    const int pl = pos_lo + r / G, h = r % G;
    row_ok[n] = pl < C;
    row_pos[n] = p0 + min(pl, C - 1);
    const size_t qrow = ((size_t)(t0 + min(pl, C - 1)) * hq_all + kvh * G + h) * D;
#pragma unroll
    for (int kk = 0; kk < S::KS; ++kk) {
      if constexpr (S::BF16) {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + qrow + kk * 32 + g * 8;
        qf[n][kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(qp));
      } else {
        qf[n][kk] = reinterpret_cast<const float*>(a.q)[qrow + kk * 4 + g];
      }
    }
  }

  f32x4 o[kRowTiles][S::DT];
  float m_run[kRowTiles], l_run[kRowTiles];
  // two-group pipeline: each row's sum of weights comes from the matrix cores,
  // as the product of an all-ones V^T fragment with the same bf16 weights PV
  // uses, rescaled like the output; every element holds the lane's row sum
  f32x4 osum[kRowTiles];
#pragma unroll
  for (int n = 0; n < kRowTiles; ++n) {
    m_run[n] = -INFINITY;
    l_run[n] = 0.f;
    osum[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) o[n][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();                                     // block-id cache ready

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.kc);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vc);
  // Pool row of logical block lb of a tile that `cached` says lies inside the
  // LDS cache (the same for the whole tile). Past the cache the row is read
  // and checked here; that read waits for itself inside its branch, so the
  // common path never waits for an outstanding K/V load.
  const __amdgpu_buffer_rsrc_t bt_rsrc = make_rsrc(bt_row, (uint32_t)a.max_blocks * 4u);
  auto block_row = [&](int lb, bool cached) -> int {
    if (cached) return bt_lds[lb - lb0];
    int r = -1;
    if (lb < nb_need) {
      if (lb >= a.max_blocks) {
        bad |= KVC_DEVERR_CONTEXT;
      } else {
        const int blk = __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, lb * 4, 0, 0);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        if ((unsigned)blk < (unsigned)a.num_blocks)
          r = blk * a.hkv + kvh;
        else
          bad |= KVC_DEVERR_BLOCK_ID;
      }
    }
    return r;
  };
  // 16 bytes (chunk c) of key `key` of tile kt. An absent key loads from the
  // pool's first row (always valid) and is zeroed when stored to LDS, so no
  // wait for the load lands here.
  struct Row16 { int64_t off; bool ok; };
  auto locate = [&](int kt, int key, bool cached) -> Row16 {
    const int r = block_row(kt * 4 + (key >> 4), cached);
    const bool ok = r >= 0 && kt * kKeyTile + key < kv_len;
    return {ok ? (int64_t)r * (16 * RB_MEM) + (key & 15) * RB_MEM : 0, ok};
  };
  auto zero_unless = [](bool ok, const u32x4& v) { return ok ? v : u32x4{0u, 0u, 0u, 0u}; };

  // Buffer->LDS staging (bf16, head dim 64 and 128): tiles go from the pool
  // straight into LDS, 1 KB per wave instruction (64 / NC keys), lane l writing
  // the 16-byte slot l % NC of its key's row. K rows hold chunk c at slot
  // c ^ (key % NC), which makes the K fragment reads (16 keys x one chunk per
  // 16 lanes) conflict-free. V rows are read by the transposing reads instead,
  // whose 16 lanes take two adjacent chunks of four consecutive keys: with the
  // K swizzle keys 2i and 2i + 1 put those chunks in the same banks, so V rows
  // hold chunk c at slot c ^ 2 (key % (NC / 2)), which gives the rows of a read
  // distinct banks. A lane fetches the chunk that belongs in its slot.
  constexpr int kKeysPerDma = 64 / S::NC;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto v_swz = [](int key) { return 2 * (key % (S::NC / 2)); };
  // V fragment read offsets inside a tile, per dim tile (see v_frag_issue)
  int v_off[S::DT];
  if constexpr (TWO) {
    const int v_row = 4 * g + (l16 >> 2);
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
      v_off[dt] = v_row * S::RB + (((2 * dt + ((l16 & 3) >> 1)) ^ v_swz(v_row)) << 4) + (l16 & 1) * 8;
  }

  // Register staging of K and V tiles for the lockstep pipeline (fp32 caches
  // and 32 dims). K runs two tiles ahead of V (QK^T of tile k+1 is computed
  // before PV of tile k), so each is loaded on its own.
  constexpr bool kAllK = S::K_UNITS % kPfThreads == 0;   // every thread has every K unit
  constexpr bool kAllV = S::V_UNITS % kPfThreads == 0;
  u32x4 kr[S::KPT], vr[S::VPT][S::VCH];
  bool kok[S::KPT], vok[S::VPT][S::VCH];
  static_assert(!F8 || TWO, "fp8 tiles are staged by the two-group pipeline only");
  // fp8 codes (8 of them) times their row's scale, rounded to bf16
  auto dequant = [](const u32x2& w, float sc) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false), d = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, true);
    return u32x4{pack_bf16x2(a[0] * sc, a[1] * sc), pack_bf16x2(b[0] * sc, b[1] * sc),
                 pack_bf16x2(c[0] * sc, c[1] * sc), pack_bf16x2(d[0] * sc, d[1] * sc)};
  };
  // A wave's K units cover 64 / NC <= 16 consecutive keys starting at a
  // multiple of 64 / NC, so they sit in one block: its base is a scalar, and
  // the lane's offset inside the block does not change between tiles. A unit
  // of an absent block reads inside the pool's first block (always valid).
  static_assert(16 % (64 / S::NC) == 0, "a wave's K rows stay in one block");
  auto load_k = [&](int kt) {
    const bool cached = 4 * (kt - t_begin) < S::BT_CACHE;
#pragma unroll
    for (int j = 0; j < S::KPT; ++j) {
      const int ci = tid + j * kPfThreads;
      const bool has = kAllK || ci < S::K_UNITS;
      const int key = has ? ci / S::NC : 0;
      const int r = __builtin_amdgcn_readfirstlane(
          block_row(kt * 4 + __builtin_amdgcn_readfirstlane(key >> 4), cached));
      const uint8_t* base = kbase + (r >= 0 ? (int64_t)r * (16 * RB_MEM) : 0);
      kok[j] = has && r >= 0 && kt * kKeyTile + key < kv_len;
      kr[j] = *reinterpret_cast<const u32x4*>(base + (key & 15) * S::RB + (ci % S::NC) * 16);
    }
  };
  auto load_v = [&](int kt) {
    const bool cached = 4 * (kt - t_begin) < S::BT_CACHE;
#pragma unroll
    for (int j = 0; j < S::VPT; ++j) {
      const int u = tid + j * kPfThreads;
      const bool has = kAllV || u < S::V_UNITS;
#pragma unroll
      for (int x = 0; x < S::VCH; ++x) {
        // bf16 unit u = (key pair u % 32, chunk u / 32): a wave's transposing
        // stores then cover all 32 key pairs and hit 64 distinct LDS banks
        const int key = !has ? 0 : S::BF16 ? 2 * (u % (kKeyTile / 2)) + x : u / S::NC;
        const int c = S::BF16 ? u / (kKeyTile / 2) : u % S::NC;
        const Row16 rw = locate(kt, key, cached);
        vok[j][x] = has && rw.ok;
        vr[j][x] = *reinterpret_cast<const u32x4*>(vbase + rw.off + c * 16);
      }
    }
  };
  auto store_k = [&](uint8_t* k_lds) {
#pragma unroll
    for (int j = 0; j < S::KPT; ++j) {
      const int ci = tid + j * kPfThreads;
      if (kAllK || ci < S::K_UNITS) {
        const int key = ci / S::NC, c = ci % S::NC;
        *reinterpret_cast<u32x4*>(k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)) =
            zero_unless(kok[j], kr[j]);
      }
    }
  };
  auto store_v = [&](uint8_t* v_lds) {
#pragma unroll
    for (int j = 0; j < S::VPT; ++j) {
      const int u = tid + j * kPfThreads;
      if (!kAllV && u >= S::V_UNITS) continue;
      const u32x4 v0 = zero_unless(vok[j][0], vr[j][0]);
      const u32x4 v1 = zero_unless(vok[j][S::VCH - 1], vr[j][S::VCH - 1]);
      if constexpr (S::BF16) {
        // keys (2kp, 2kp+1) x dims 8c..8c+7 -> V^T[dim][2kp .. 2kp+1], one dword per dim
        const int kp = u % (kKeyTile / 2), c = u / (kKeyTile / 2);
        uint32_t* vt = reinterpret_cast<uint32_t*>(v_lds);
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const uint32_t lo = __builtin_amdgcn_perm(v1[wd], v0[wd], 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(v1[wd], v0[wd], 0x07060302u);
          vt[((c * 8 + 2 * wd) * S::VT_STRIDE + 2 * kp) / 2] = lo;
          vt[((c * 8 + 2 * wd + 1) * S::VT_STRIDE + 2 * kp) / 2] = hi;
        }
      } else {
        const int key = u / S::NC, c = u % S::NC;
        *reinterpret_cast<u32x4*>(v_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)) = v0;
      }
    }
  };

  // ---- S^T = K . Q^T for one key tile: 4 key tiles x kRowTiles row tiles.
  // The K fragments of key tile m+1 are read from LDS while tile m multiplies.
  auto load_kf = [&](const uint8_t* k_lds, int m, Frag (&kf)[S::KS]) {
    const int key = m * 16 + l16;
#pragma unroll
    for (int kk = 0; kk < S::KS; ++kk) {
      if constexpr (S::BF16) {
        const int c = kk * 4 + g;
        kf[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                                                  k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)));
      } else {
        const int c = kk;                            // dims 4kk .. 4kk+3, element g
        kf[kk] = *reinterpret_cast<const float*>(k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4) +
                                                 g * 4);
      }
    }
  };
  auto qk = [&](const uint8_t* k_lds, f32x4 (&sacc)[4][kRowTiles]) {
    if constexpr (S::BF16) {
      // steps (m, kk); the fragment of step st+kAhead is read while step st
      // multiplies, and a scheduling fence per step keeps that order
      constexpr int kSteps = 4 * S::KS, kAhead = 3;
      bf16x8_t kf[kAhead + 1];
      auto frag = [&](int st) {
        const int key = (st / S::KS) * 16 + l16, c = (st % S::KS) * 4 + g;
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                                                k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)));
      };
#pragma unroll
      for (int st = 0; st < kAhead; ++st) kf[st] = frag(st);
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        if (st + kAhead < kSteps) kf[(st + kAhead) % (kAhead + 1)] = frag(st + kAhead);
        const int m = st / S::KS, kk = st % S::KS;
#pragma unroll
        for (int n = 0; n < kRowTiles; ++n)
          sacc[m][n] = M::mma(kf[st % (kAhead + 1)], qf[n][kk],
                              kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[m][n]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        Frag kf[S::KS];
        load_kf(k_lds, m, kf);
#pragma unroll
        for (int kk = 0; kk < S::KS; ++kk)
#pragma unroll
          for (int n = 0; n < kRowTiles; ++n)
            sacc[m][n] = M::mma(kf[kk], qf[n][kk], kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[m][n]);
      }
    }
  };
  // causal mask, only for tiles that reach past the smallest row position
  auto mask = [&](f32x4 (&sacc)[4][kRowTiles], int key0) {
    if (__builtin_expect(key0 + kKeyTile - 1 > p0 + pos_lo, 0)) {
#pragma unroll
      for (int n = 0; n < kRowTiles; ++n)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key0 + m * 16 + g * 4 + i > row_pos[n]) sacc[m][n][i] = -INFINITY;
    }
  };
  // ---- online softmax of one tile (lane owns row l16 of each row tile).
  // Row sums stay per lane (a partial over this lane's keys) until the end;
  // the running max is reduced across the row every tile.
  using PTile = typename PfP<S::BF16>::Tile;
  auto softmax = [&](const f32x4 (&sacc)[4][kRowTiles], PTile& pt, float (&alpha)[kRowTiles]) {
#pragma unroll
    for (int n = 0; n < kRowTiles; ++n) {
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[m][n][i]);
      mx = rows_max(mx);
      const float m_new = fmaxf(m_run[n], mx * a.scale_log2);
      const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
      alpha[n] = __builtin_amdgcn_exp2f(m_run[n] - m_safe);
      m_run[n] = m_new;
      float p[4][4];
      float rs = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[m][i] = __builtin_amdgcn_exp2f(fmaf(sacc[m][n][i], a.scale_log2, -m_safe));
          if constexpr (!S::BF16) rs += p[m][i];
        }
      if constexpr (S::BF16) {
        // the row sum adds the bf16 weights the PV product uses (in the
        // two-group pipeline the matrix cores add them)
#pragma unroll
        for (int mp = 0; mp < 2; ++mp) {
          pt.v[mp][n] = u32x4{pack_bf16x2(p[2 * mp][0], p[2 * mp][1]),
                              pack_bf16x2(p[2 * mp][2], p[2 * mp][3]),
                              pack_bf16x2(p[2 * mp + 1][0], p[2 * mp + 1][1]),
                              pack_bf16x2(p[2 * mp + 1][2], p[2 * mp + 1][3])};
          if constexpr (!TWO) {
#pragma unroll
            for (int q = 0; q < 4; ++q) rs = dot2_bf16(pt.v[mp][n][q], kBf16OnePair, rs);
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) pt.v[m][n][i] = p[m][i];
      }
      if constexpr (!TWO) l_run[n] = fmaf(l_run[n], alpha[n], rs);
    }
  };
  // ---- V fragment (MFMA A operand of O^T += V^T . P^T) for key pair mp and
  // dim tile dt: keys 32mp + 4g + 0..3 and 32mp + 16 + 4g + 0..3 of dim
  // 16dt + l16, in the key order of the S^T accumulators. Read as two
  // 8-byte halves; v_frag_use joins them.
  struct VHalves { u32x2 lo, hi; };
  auto v_frag_issue = [&](const uint8_t* v_lds, int mp, int dt) -> VHalves {
    if constexpr (TWO) {
      // row-major tile: each transposing read gathers 4 keys x 16 dims over a
      // 16-lane group; lane i of the group addresses key 4g + i/4, dims
      // 16dt + 4(i%4) .. +3 (chunk swizzle of that key's row applied)
      // (the key offset is an immediate, so both key pairs share one address)
      const uint32_t p = (uint32_t)(uintptr_t)(lds_void*)v_lds + (uint32_t)v_off[dt];
      if (mp == 0) return {tr_read_b64<0>(p), tr_read_b64<16 * S::RB>(p)};
      return {tr_read_b64<32 * S::RB>(p), tr_read_b64<48 * S::RB>(p)};
    } else {
      const uint16_t* rowp =
          reinterpret_cast<const uint16_t*>(v_lds) + (dt * 16 + l16) * S::VT_STRIDE + mp * 32 + g * 4;
      return {*reinterpret_cast<const u32x2*>(rowp), *reinterpret_cast<const u32x2*>(rowp + 16)};
    }
  };
  auto v_frag_use = [&](const VHalves& f) -> bf16x8_t {
    return __builtin_bit_cast(bf16x8_t, u32x4{f.lo[0], f.lo[1], f.hi[0], f.hi[1]});
  };
  // ---- O^T += V^T . P^T for one tile; V fragments are read one step ahead
  auto pv = [&](const uint8_t* v_lds, const PTile& pt) {
    if constexpr (S::BF16) {
      VHalves vf[2];
      vf[0] = v_frag_issue(v_lds, 0, 0);
#pragma unroll
      for (int st = 0; st < 2 * S::DT; ++st) {          // st = (mp, dt)
        const int mp = st / S::DT, dt = st % S::DT;
        const bool more = st + 1 < 2 * S::DT;
        if (more) vf[(st + 1) & 1] = v_frag_issue(v_lds, (st + 1) / S::DT, (st + 1) % S::DT);
        const bf16x8_t a = v_frag_use(vf[st & 1]);
#pragma unroll
        for (int n = 0; n < kRowTiles; ++n)
          o[n][dt] = M::mma(a, __builtin_bit_cast(bf16x8_t, pt.v[mp][n]), o[n][dt]);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = m * 16 + g * 4 + i;
#pragma unroll
          for (int dt = 0; dt < S::DT; ++dt) {
            const int dim = dt * 16 + l16, c = dim >> 2;
            const float vf = *reinterpret_cast<const float*>(
                v_lds + key * S::RB + ((c ^ (key % S::NC)) << 4) + (dim & 3) * 4);
#pragma unroll
            for (int n = 0; n < kRowTiles; ++n) o[n][dt] = M::mma(vf, pt.v[m][n][i], o[n][dt]);
          }
        }
    }
  };
  // bf16: PV of one tile fused with the softmax of the next, one PV step
  // (a V fragment times both row tiles) at a time with a slice of the softmax
  // after it, each step fenced so the vector work stays between the MFMAs.
  // Softmax units: 0, 1 = partial row max of row tile 0, 1; 2 = max across
  // the row, new running max and rescale factor; 3 + e = weight e (row tile
  // e / 16, key tile (e / 4) % 4, element e % 4), packed to bf16 in pairs.
  auto pv_softmax = [&](const uint8_t* v_lds, const PTile& pt, const f32x4 (&sc)[4][kRowTiles],
                        PTile& pn, float (&alpha)[kRowTiles]) {
    if constexpr (S::BF16) {
      constexpr int kSteps = 2 * S::DT, kAhead = 2;
      constexpr int kUnits = 3 + 16 * kRowTiles;
      auto frag = [&](int st) { return v_frag_issue(v_lds, st / S::DT, st % S::DT); };
      float mx[kRowTiles], msafe[kRowTiles], rs[kRowTiles], pw[kRowTiles][4][4];
      auto unit = [&](int u) {
        if (u < kRowTiles) {
          float v = -INFINITY;
  #pragma unroll
          for (int m = 0; m < 4; ++m)
  #pragma unroll
            for (int i = 0; i < 4; ++i) v = fmaxf(v, sc[m][u][i]);
          mx[u] = v;
        } else if (u == kRowTiles) {
  #pragma unroll
          for (int n = 0; n < kRowTiles; ++n) {
            const float m_new = fmaxf(m_run[n], rows_max(mx[n]) * a.scale_log2);
            msafe[n] = (m_new == -INFINITY) ? 0.f : m_new;
            alpha[n] = __builtin_amdgcn_exp2f(m_run[n] - msafe[n]);
            m_run[n] = m_new;
            rs[n] = 0.f;
          }
        } else {
          const int e = u - kRowTiles - 1, n = e / 16, m = (e / 4) % 4, i = e % 4;
          pw[n][m][i] = __builtin_amdgcn_exp2f(fmaf(sc[m][n][i], a.scale_log2, -msafe[n]));
          if (i & 1) {
            const uint32_t pair = pack_bf16x2(pw[n][m][i - 1], pw[n][m][i]);
            pn.v[m / 2][n][(m % 2) * 2 + i / 2] = pair;
            rs[n] = dot2_bf16(pair, kBf16OnePair, rs[n]);   // sum of the weights PV uses
          }
        }
      };
      VHalves vf[kAhead + 1];
  #pragma unroll
      for (int st = 0; st < kAhead; ++st) vf[st] = frag(st);
  #pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        if (st + kAhead < kSteps) vf[(st + kAhead) % (kAhead + 1)] = frag(st + kAhead);
        const int mp = st / S::DT, dt = st % S::DT;
        const bf16x8_t va = v_frag_use(vf[st % (kAhead + 1)]);
  #pragma unroll
        for (int n = 0; n < kRowTiles; ++n)
          o[n][dt] = M::mma(va, __builtin_bit_cast(bf16x8_t, pt.v[mp][n]), o[n][dt]);
  #pragma unroll
        for (int u = 0; u < kUnits; ++u)
          if (u * kSteps / kUnits == st) unit(u);
        __builtin_amdgcn_sched_barrier(0);
      }
  #pragma unroll
      for (int n = 0; n < kRowTiles; ++n) l_run[n] = fmaf(l_run[n], alpha[n], rs[n]);
    }
  };
  auto rescale = [&](const float (&alpha)[kRowTiles]) {
#pragma unroll
    for (int n = 0; n < kRowTiles; ++n)
      if (__builtin_expect(__any(alpha[n] != 1.f), 0)) {   // wave-uniform: skip when no max moved
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) o[n][dt] *= alpha[n];
        if constexpr (TWO) osum[n] *= alpha[n];
      }
  };

  // Barrier for LDS hand-off only: waits for this wave's LDS operations, not
  // for its outstanding global loads (which a full fence would drain).
  auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // Software pipeline over key tiles. Iteration kt holds K(kt+1) and V(kt) in
  // LDS and P(kt) in registers: it multiplies QK^T of tile kt+1 on MFMA, then
  // PV of tile kt on MFMA while the softmax of tile kt+1 runs on the vector
  // ALUs, and applies tile kt+1's rescale after PV(kt). K(kt+2) and V(kt+1)
  // are loaded during the iteration and stored behind it; K and V each have
  // two LDS buffers, and the barrier closing an iteration publishes the new
  // tiles after every wave has finished with the ones they overwrite.
  f32x4 sacc[4][kRowTiles];
  PTile pt;
  float alpha[kRowTiles];
  // the next tile's weights and row sums are computed between the PV MFMAs;
  // pin them there so they are not sunk past the rescale branch
  auto pin = [&](PTile& pn) {
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
      for (int n = 0; n < kRowTiles; ++n) asm volatile("" : "+v"(pn.v[mp][n]));
#pragma unroll
    for (int n = 0; n < kRowTiles; ++n) asm volatile("" : "+v"(l_run[n]));
  };
  if constexpr (TWO) {
    // Two groups of four waves with one wave of each on every SIMD (waves w
    // and w + 4 share a SIMD). Each group alternates a matrix half-step
    // (QK^T of tile k and PV of tile k - 1: 64 MFMAs, fragments from LDS)
    // and a vector half-step (the softmax of tile k, the rescale, and its
    // share of the tile staging), and group 1 runs one half-step behind
    // group 0: on every SIMD one wave's MFMAs run while the other wave's
    // vector work does. A workgroup barrier closes every half-step.
    //   half-step 2k:   group 0 matrix(k),      group 1 vector(k - 1)
    //   half-step 2k+1: group 0 vector(k),      group 1 matrix(k)
    // K(k) and V(k) sit in buffer k % NB. Group 1 stages K tiles, group 0 V
    // tiles, wave i of a group block i of the tile (16 keys). In vector(k)
    // group 1 issues K(k + NB) (into the buffer K(k) left at half-step
    // 2k + 1) and group 0 V(k + NB - 2) (V(k - 2) was last read at 2k - 1);
    // at the end of every vector half-step a wave waits for its batch issued
    // NB - 2 vector half-steps earlier, which the next matrix half-steps read
    // (K(k + 2) from 2k + 4, V(k) from 2k + 2): every batch has NB - 2
    // iterations to land.
    constexpr int NB = S::NBUF;
    constexpr int BPB = S::BPB;
    const int grp = wu >> 2, wi = wu & 3;
    const int n_t = t_end - t_begin;
    auto kbuf = [&](int k) { return smem + (k % NB) * S::K_LDS; };
    auto vbuf = [&](int k) { return smem + (NB + k % NB) * S::K_LDS; };
    // lane l of load j writes the 16-byte slot l % NC of key j * 64/NC + l / NC
    // of the block, so it fetches the chunk the tile's swizzle puts there
    uint32_t blk_voff[BPB];
#pragma unroll
    for (int j = 0; j < BPB; ++j) {
      const int kb = j * kKeysPerDma + lane / S::NC, key = wi * 16 + kb;
      const int swz = grp == 1 ? key % S::NC : v_swz(key);   // group 1 stages K, group 0 V
      blk_voff[j] = (uint32_t)(kb * S::RB + (((lane % S::NC) ^ swz) << 4));
    }
    // block wi of tile k of `pool` into `lds`; keys past the sequence and
    // blocks that hold none read as zeros (the buffer range check)
    auto stage = [&](int k, const uint8_t* pool, uint8_t* lds) {
      const int kt = t_begin + k;
      const int r = __builtin_amdgcn_readfirstlane(block_row(kt * 4 + wi, 4 * k < S::BT_CACHE));
      const uint8_t* base = pool + (r >= 0 ? (int64_t)r * (16 * S::RB) : 0);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, r >= 0 ? 16u * S::RB : 0u);
      const int key0 = kt * kKeyTile + wi * 16;
      const bool edge = key0 + 16 > kv_len;
#pragma unroll
      for (int j = 0; j < BPB; ++j) {
        uint32_t voff = blk_voff[j];
        if (edge && key0 + j * kKeysPerDma + lane / S::NC >= kv_len) voff = kDmaPastEnd;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (wi * BPB + j) * 1024), 16,
                                                 voff, 0, 0, 0);
      }
    };
    // fp8: the same tiles staged through registers. A wave reads its block of
    // a tile (codes and row scales; the chunk order the swizzle puts in each
    // lane's 16-byte slot) in one vector half-step and writes it, converted
    // to bf16, lane after lane in its next one. An absent block reads inside
    // the pool's first block; it and keys past the sequence are written as
    // zeros.
    u32x2 st_codes[BPB];
    float st_scale[BPB];
    bool st_ok[BPB];
    auto fetch8 = [&](int k, const uint8_t* pool, const float* scales) {
      const int kt = t_begin + k;
      const int r = __builtin_amdgcn_readfirstlane(block_row(kt * 4 + wi, 4 * k < S::BT_CACHE));
      const uint8_t* base = pool + (r >= 0 ? (int64_t)r * (16 * RB_MEM) : 0);
      const float* sc = scales + (r >= 0 ? (int64_t)r * 16 : 0);
      const int key0 = kt * kKeyTile + wi * 16;
#pragma unroll
      for (int j = 0; j < BPB; ++j) {
        const int kb = j * kKeysPerDma + lane / S::NC, key = wi * 16 + kb;
        const int swz = grp == 1 ? key % S::NC : v_swz(key);
        st_codes[j] = *reinterpret_cast<const u32x2*>(base + kb * RB_MEM + (((lane % S::NC) ^ swz) << 3));
        st_scale[j] = sc[kb];
        st_ok[j] = r >= 0 && key0 + kb < kv_len;
      }
    };
    auto put8 = [&](uint8_t* lds) {
#pragma unroll
      for (int j = 0; j < BPB; ++j)
        *reinterpret_cast<u32x4*>(lds + (wi * BPB + j) * 1024 + lane * 16) =
            zero_unless(st_ok[j], dequant(st_codes[j], st_scale[j]));
    };
    // fp8 tiles ahead of their use: at vector(k) group 1 writes K(k + NB - 1)
    // (into the buffer K(k - 1) left at half-step 2k - 1; read from 2k + 2NB - 2)
    // and group 0 V(k + NB - 3) (V(k - 3) was last read at 2k - 3; read from
    // 2k + 4), then each reads the next tile of its kind into registers
    const int put_lead = grp == 1 ? NB - 1 : NB - 3;

    // end of a half-step: this wave's LDS reads are done and, if `wait`, at
    // most `newer` of its staging batches are still in flight; then the barrier
    static_assert(NB >= 3 && NB <= 4, "newer batches: 0 .. 2");
    auto half_step_end = [](bool wait, int newer) {
      if (!wait)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (newer >= 2)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * S::BPB) : "memory");
      else if (newer == 1)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(S::BPB) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // staging batches a wave issued after the one it waits for at the end of
    // vector(k): K(k + 3 .. k + NB) for group 1 (it waits for K(k + 2)),
    // V(k + 1 .. k + NB - 2) for group 0 (it waits for V(k)); k = -1: the prologue
    auto newer_batches = [&](int k) {
      const int first = grp == 1 ? k + 3 : k + 1, last = grp == 1 ? k + NB : k + NB - 2;
      return max(0, min(last, n_t - 1) - first + 1);
    };
    // matrix half-step: QK^T of tile k (QK) and PV of tile k - 1 (PV), one
    // QK^T step and one PV step at a time (each both row tiles), K fragments
    // read three steps ahead and V fragments two
    auto matrix = [&](auto qk_tag, auto pv_tag, int k) {
      constexpr bool QK = decltype(qk_tag)::value, PV = decltype(pv_tag)::value;
      constexpr int kQ = 4 * S::KS, kP = 2 * S::DT;      // steps of each product
      constexpr int kSteps = QK ? kQ : kP;
      static_assert(!QK || !PV || kQ == kP, "the two products interleave step for step");
      const uint8_t* kl = kbuf(k);
      const uint8_t* vl = vbuf(k + NB - 1);              // tile k - 1
      bf16x8_t kf[4];
      auto kfrag = [&](int st) {
        const int key = (st / S::KS) * 16 + l16, c = (st % S::KS) * 4 + g;
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                                                kl + key * S::RB + ((c ^ (key % S::NC)) << 4)));
      };
      VHalves vf[3];
      if constexpr (QK) {
#pragma unroll
        for (int st = 0; st < 3; ++st) kf[st] = kfrag(st);
      }
      if constexpr (PV) {
        vf[0] = v_frag_issue(vl, 0, 0);
        vf[1] = v_frag_issue(vl, 1 / S::DT, 1 % S::DT);
      }
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        if constexpr (QK) {
          if (st + 3 < kQ) kf[(st + 3) % 4] = kfrag(st + 3);
          const int m = st / S::KS, kk = st % S::KS;
#pragma unroll
          for (int nn = 0; nn < kRowTiles; ++nn)
            sacc[m][nn] = M::mma(kf[st % 4], qf[nn][kk], kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[m][nn]);
        }
        if constexpr (PV) {
          if (st + 2 < kP) vf[(st + 2) % 3] = v_frag_issue(vl, (st + 2) / S::DT, (st + 2) % S::DT);
          const bf16x8_t va = v_frag_use(vf[st % 3]);
          const int mp = st / S::DT, dt = st % S::DT;
#pragma unroll
          for (int nn = 0; nn < kRowTiles; ++nn)
            o[nn][dt] = M::mma(va, __builtin_bit_cast(bf16x8_t, pt.v[mp][nn]), o[nn][dt]);
          if (dt == S::DT - 1) {
            const bf16x8_t ones = __builtin_bit_cast(
                bf16x8_t, u32x4{kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair});
#pragma unroll
            for (int nn = 0; nn < kRowTiles; ++nn)
              osum[nn] = M::mma(ones, __builtin_bit_cast(bf16x8_t, pt.v[mp][nn]), osum[nn]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // vector half-step: softmax of tile k, the rescale of the accumulators,
    // this wave's staging batch and the wait for its older one
    auto vector = [&](int k) {
      mask(sacc, (t_begin + k) * kKeyTile);
      softmax(sacc, pt, alpha);
      rescale(alpha);
      // one call site, its pool, buffer and tile chosen by selects (two call
      // sites, one per group, were merged by the compiler into a block that
      // left the K pool's base unset on group 1's path)
      if constexpr (F8) {
        const int kp = k + put_lead;
        if (kp < n_t) put8(grp == 1 ? kbuf(kp) : vbuf(kp));
        if (kp + 1 < n_t) fetch8(kp + 1, grp == 1 ? kbase : vbase, grp == 1 ? a.ks : a.vs);
        half_step_end(false, 0);
      } else {
        const int ks = grp == 1 ? k + NB : k + NB - 2;
        if (ks < n_t) stage(ks, grp == 1 ? kbase : vbase, grp == 1 ? kbuf(ks) : vbuf(ks));
        half_step_end(true, newer_batches(k));
      }
    };

    // prologue: K(0 .. NB-1) by group 1, V(0 .. NB-3) by group 0; K(0) and
    // K(1) must have landed before the first matrix half-steps
    if constexpr (F8) {
      // fp8: K(0 .. NB-2) by group 1, V(0 .. NB-4) by group 0 written now,
      // the next tile of each kind read into registers
      for (int k = 0; k < min(put_lead, n_t); ++k) {
        fetch8(k, grp == 1 ? kbase : vbase, grp == 1 ? a.ks : a.vs);
        put8(grp == 1 ? kbuf(k) : vbuf(k));
      }
      if (put_lead < n_t) fetch8(put_lead, grp == 1 ? kbase : vbase, grp == 1 ? a.ks : a.vs);
      half_step_end(false, 0);
    } else {
      const int n_pro = min(grp == 1 ? NB : NB - 2, n_t);
      for (int k = 0; k < n_pro; ++k) stage(k, grp == 1 ? kbase : vbase, grp == 1 ? kbuf(k) : vbuf(k));
      half_step_end(grp == 1, newer_batches(-1));      // group 1: K(2 .. NB-1) may stay in flight
    }
    if (grp == 1) half_step_end(false, 0);            // half-step 0: group 1 idle
    matrix(std::true_type{}, std::false_type{}, 0);
    half_step_end(false, 0);
    vector(0);
    for (int k = 1; k < n_t; ++k) {
      matrix(std::true_type{}, std::true_type{}, k);
      half_step_end(false, 0);
      vector(k);
    }
    matrix(std::false_type{}, std::true_type{}, n_t);
    half_step_end(false, 0);
    if (grp == 0) half_step_end(false, 0);            // last half-step: group 0 idle
  } else {
  auto kbuf = [&](int i) { return smem + (i & 1) * S::K_LDS; };
  auto vbuf = [&](int i) { return smem + 2 * S::K_LDS + (i & 1) * S::V_LDS; };
  load_k(t_begin);
  load_v(t_begin);
  store_k(kbuf(t_begin));
  store_v(vbuf(t_begin));
  if (t_end - t_begin > 1) {
    load_k(t_begin + 1);
    store_k(kbuf(t_begin + 1));
  }
  lds_barrier();
  qk(kbuf(t_begin), sacc);
  mask(sacc, t_begin * kKeyTile);
  softmax(sacc, pt, alpha);                           // o is still zero: no rescale
  lds_barrier();                                       // K(0) read by every wave
  for (int kt = t_begin; kt + 1 < t_end; ++kt) {
    const bool more_k = kt + 2 < t_end;
    if (more_k) load_k(kt + 2);
    load_v(kt + 1);
    qk(kbuf(kt + 1), sacc);
    mask(sacc, (kt + 1) * kKeyTile);
    PTile pt_next;
    if constexpr (S::BF16) {
      pv_softmax(vbuf(kt), pt, sacc, pt_next, alpha);
      pin(pt_next);
    } else {
      pv(vbuf(kt), pt);
      softmax(sacc, pt_next, alpha);
    }
    rescale(alpha);
    pt = pt_next;
    if (more_k) store_k(kbuf(kt));
    store_v(vbuf(kt + 1));
    lds_barrier();
  }
  pv(vbuf(t_end - 1), pt);
  }

  if (bad) flag_error(a.err, bad);

  // ---- write rows: lane holds dims 16dt + 4g .. +3 of row l16 ----
  float l_row[kRowTiles];
#pragma unroll
  for (int n = 0; n < kRowTiles; ++n)
    l_row[n] = TWO ? osum[n][0] : rows_sum(l_run[n]);   // whole wave, before any exit
#pragma unroll
  for (int n = 0; n < kRowTiles; ++n) {
    if (!row_ok[n]) continue;
    const int r = w * (kRowTiles * 16) + n * 16 + l16;
    const int pl = pos_lo + r / G, h = r % G;
    const size_t row = (size_t)(t0 + pl) * hq_all + kvh * G + h;
    if (a.n_split == 1) {
      const float inv = 1.f / l_row[n];
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) store4<CT>(a.out, row * D + dt * 16 + g * 4, o[n][dt], inv);
    } else {
      // partial of this key range: unnormalised accumulators, running max, row sum
      const size_t pr = row * a.n_split + sp;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt)
        *reinterpret_cast<f32x4*>(a.ws_o + pr * D + dt * 16 + g * 4) = o[n][dt];
      if (g == 0) a.ws_ml[pr] = float2{m_run[n], l_row[n]};
    }
  }
}

}  // namespace kvc
