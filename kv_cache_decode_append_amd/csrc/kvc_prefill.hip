// Chunked-prefill attention: write a prompt chunk's K/V into the paged cache,
// then causal attention of every chunk position over the cached prefix and the
// chunk's own positions up to itself.
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
// Tiling (one workgroup = 4 waves = 128 query rows of one kv head):
//   row r <-> (position qt*MP + r / G, query head kvh*G + r % G), MP = 128 / G,
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

#include <math.h>

#include "kvc_append.h"
#include "kvc_device.h"
#include "kvc_host.h"

namespace kvc {

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kRowTiles = 2;                        // 16-row tiles per wave
constexpr int kRows = kPfWaves * kRowTiles * 16;    // 256 query rows per workgroup
constexpr int kKeyTile = 64;                        // keys per staged tile
constexpr int kBtCache = 2048;                      // block ids kept in LDS (32,768 keys)

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
  static constexpr int BUF = K_LDS + V_LDS;         // one staged key tile
  static constexpr int SMEM = 2 * BUF + kBtCache * 4;
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
  int32_t n_work;     // n_qt * hkv * n_seqs
  float scale_log2;
};

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

template <typename T, int D, int G>
__global__ __launch_bounds__(kPfThreads) void prefill_attention_kernel(PrefillArgs a) {
  using S = PfShape<T, D, G>;
  using M = PfMfma<T>;
  using Frag = typename M::Frag;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::SMEM];
  int32_t* bt_lds = reinterpret_cast<int32_t*>(smem + 2 * S::BUF);

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so give
  // each XCD a contiguous run of work items; the query tiles of one (sequence,
  // kv head) then share one L2 while they sweep the same keys.
  const int per_xcd = gridDim.x / 8;
  const int work = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (work >= a.n_work) return;
  const int qt = work % a.n_qt;
  const int kvh = (work / a.n_qt) % a.hkv;
  const int s = work / (a.n_qt * a.hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int t0 = a.cu[s];
  const int C = a.cu[s + 1] - t0;
  const int p0 = a.prefix[s];
  const int pos_lo = qt * S::MP;
  if (!chunk_ok(t0, C, p0, a.total, a.max_chunk)) {
    if (qt == 0 && kvh == 0 && tid == 0) flag_error(a.err, KVC_DEVERR_CONTEXT);
    return;
  }
  if (pos_lo >= C) return;
  const int kv_len = p0 + C;                           // keys that exist after the write
  const int last_pos = p0 + min(pos_lo + S::MP, C) - 1;
  const int n_tiles = last_pos / kKeyTile + 1;
  const int hq_all = a.hkv * G;
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;

  // block ids of the keys this workgroup reads, cached in LDS
  const int nb_need = (min(kv_len, n_tiles * kKeyTile) + 15) / 16;
  for (int i = tid; i < min(nb_need, kBtCache); i += kPfThreads)
    bt_lds[i] = i < a.max_blocks ? bt_row[i] : -1;

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
#pragma unroll
  for (int n = 0; n < kRowTiles; ++n) {
    m_run[n] = -INFINITY;
    l_run[n] = 0.f;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) o[n][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();                                     // block-id cache ready

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.kc);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vc);
  // byte offset of token `key` (row start) of this kv head, or -1 when absent;
  // contract violations are collected per lane and flagged once at the end
  int bad = 0;
  auto row_off = [&](int key) -> int64_t {
    const int lb = key >> 4;
    const bool in_table = lb < a.max_blocks;
    const int blk = !in_table ? -1 : (lb < kBtCache ? bt_lds[lb] : bt_row[lb]);
    const bool ok_blk = (unsigned)blk < (unsigned)a.num_blocks;
    if (key < kv_len) bad |= !in_table ? KVC_DEVERR_CONTEXT : (!ok_blk ? KVC_DEVERR_BLOCK_ID : 0);
    return (key < kv_len && ok_blk) ? (((int64_t)blk * a.hkv + kvh) * 16 + (key & 15)) * S::RB
                                    : (int64_t)-1;
  };
  // an absent row loads from the pool's first row (always valid) and is zeroed
  auto load_row16 = [&](const uint8_t* base, int64_t off, int c) -> u32x4 {
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + (off >= 0 ? off : 0) + c * 16);
    return off >= 0 ? v : u32x4{0u, 0u, 0u, 0u};
  };

  // Register staging of one key tile: issued one tile ahead so the global
  // loads overlap the MFMA work of the current tile.
  u32x4 kr[S::KPT], vr[S::VPT][S::VCH];
  auto load_tile = [&](int kt) {
    const int key0 = kt * kKeyTile;
#pragma unroll
    for (int j = 0; j < S::KPT; ++j) {
      const int ci = tid + j * kPfThreads;
      kr[j] = u32x4{0u, 0u, 0u, 0u};
      if (ci < S::K_UNITS) kr[j] = load_row16(kbase, row_off(key0 + ci / S::NC), ci % S::NC);
    }
#pragma unroll
    for (int j = 0; j < S::VPT; ++j) {
      const int u = tid + j * kPfThreads;
#pragma unroll
      for (int x = 0; x < S::VCH; ++x) {
        vr[j][x] = u32x4{0u, 0u, 0u, 0u};
        if (u < S::V_UNITS) {
          // bf16 unit u = (key pair u % 32, chunk u / 32): a wave's transposing
          // stores then cover all 32 key pairs and hit 64 distinct LDS banks
          const int key = S::BF16 ? 2 * (u % (kKeyTile / 2)) + x : u / S::NC;
          const int c = S::BF16 ? u / (kKeyTile / 2) : u % S::NC;
          vr[j][x] = load_row16(vbase, row_off(key0 + key), c);
        }
      }
    }
  };
  auto store_tile = [&](uint8_t* k_lds, uint8_t* v_lds) {
#pragma unroll
    for (int j = 0; j < S::KPT; ++j) {
      const int ci = tid + j * kPfThreads;
      if (ci < S::K_UNITS) {
        const int key = ci / S::NC, c = ci % S::NC;
        *reinterpret_cast<u32x4*>(k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)) = kr[j];
      }
    }
#pragma unroll
    for (int j = 0; j < S::VPT; ++j) {
      const int u = tid + j * kPfThreads;
      if (u >= S::V_UNITS) continue;
      if constexpr (S::BF16) {
        // keys (2kp, 2kp+1) x dims 8c..8c+7 -> V^T[dim][2kp .. 2kp+1], one dword per dim
        const int kp = u % (kKeyTile / 2), c = u / (kKeyTile / 2);
        uint32_t* vt = reinterpret_cast<uint32_t*>(v_lds);
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const uint32_t lo = __builtin_amdgcn_perm(vr[j][1][wd], vr[j][0][wd], 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(vr[j][1][wd], vr[j][0][wd], 0x07060302u);
          vt[((c * 8 + 2 * wd) * S::VT_STRIDE + 2 * kp) / 2] = lo;
          vt[((c * 8 + 2 * wd + 1) * S::VT_STRIDE + 2 * kp) / 2] = hi;
        }
      } else {
        const int key = u / S::NC, c = u % S::NC;
        *reinterpret_cast<u32x4*>(v_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)) = vr[j][0];
      }
    }
  };

  // Two LDS tile buffers: tile kt+1 is loaded during tile kt's MFMA work and
  // stored into the other buffer right after it, so one barrier per tile both
  // publishes tile kt+1 and frees tile kt's buffer.
  load_tile(0);
  store_tile(smem, smem + S::K_LDS);
  __syncthreads();
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int key0 = kt * kKeyTile;
    uint8_t* k_lds = smem + (kt & 1) * S::BUF;
    uint8_t* v_lds = k_lds + S::K_LDS;
    if (kt + 1 < n_tiles) load_tile(kt + 1);           // in flight during this tile's MFMA

    // ---- S^T = K . Q^T : 4 key tiles x kRowTiles row tiles ----
    f32x4 sacc[4][kRowTiles];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < kRowTiles; ++n) sacc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int key = m * 16 + l16;
#pragma unroll
      for (int kk = 0; kk < S::KS; ++kk) {
        Frag kf;
        if constexpr (S::BF16) {
          const int c = kk * 4 + g;
          kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                                                k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)));
        } else {
          const int c = kk;                          // dims 4kk .. 4kk+3, element g
          kf = *reinterpret_cast<const float*>(k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4) +
                                               g * 4);
        }
#pragma unroll
        for (int n = 0; n < kRowTiles; ++n) sacc[m][n] = M::mma(kf, qf[n][kk], sacc[m][n]);
      }
    }

    // ---- online softmax per row (lane owns row l16 of each row tile) ----
    // Only tiles that reach past the smallest row position need the causal mask.
    if (key0 + kKeyTile - 1 > p0 + pos_lo) {
#pragma unroll
      for (int n = 0; n < kRowTiles; ++n)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key0 + m * 16 + g * 4 + i > row_pos[n]) sacc[m][n][i] = -INFINITY;
    }
    float pbuf[4][kRowTiles][4];
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
      const float alpha = __builtin_amdgcn_exp2f(m_run[n] - m_safe);
      float rs = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[m][n][i], a.scale_log2, -m_safe));
          pbuf[m][n][i] = p;
          rs += p;
        }
      rs = rows_sum(rs);
      l_run[n] = l_run[n] * alpha + rs;
      m_run[n] = m_new;
      if (__builtin_expect(__any(alpha != 1.f), 0)) {   // wave-uniform: skip when no max moved
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) o[n][dt] *= alpha;
      }
    }

    // ---- O^T += V^T . P^T ----
    if constexpr (S::BF16) {
      const uint16_t* vt = reinterpret_cast<const uint16_t*>(v_lds);
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) {                 // key tiles (2mp, 2mp+1) = 32 keys
        Frag pf[kRowTiles];
#pragma unroll
        for (int n = 0; n < kRowTiles; ++n) {
          const float* a0 = pbuf[2 * mp][n];
          const float* a1 = pbuf[2 * mp + 1][n];
          const u32x4 pk = u32x4{pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]),
                                 pack_bf16x2(a1[0], a1[1]), pack_bf16x2(a1[2], a1[3])};
          pf[n] = __builtin_bit_cast(bf16x8_t, pk);
        }
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) {
          const uint16_t* rowp = vt + (dt * 16 + l16) * S::VT_STRIDE + mp * 32 + g * 4;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(rowp);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(rowp + 16);
          const Frag vf = __builtin_bit_cast(bf16x8_t, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int n = 0; n < kRowTiles; ++n) o[n][dt] = M::mma(vf, pf[n], o[n][dt]);
        }
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
            for (int n = 0; n < kRowTiles; ++n) o[n][dt] = M::mma(vf, pbuf[m][n][i], o[n][dt]);
          }
        }
    }
    if (kt + 1 < n_tiles) {
      uint8_t* nk = smem + ((kt + 1) & 1) * S::BUF;
      store_tile(nk, nk + S::K_LDS);
    }
    __syncthreads();
  }

  if (bad) flag_error(a.err, bad);

  // ---- write rows: lane holds dims 16dt + 4g .. +3 of row l16 ----
#pragma unroll
  for (int n = 0; n < kRowTiles; ++n) {
    if (!row_ok[n]) continue;
    const int r = w * (kRowTiles * 16) + n * 16 + l16;
    const int pl = pos_lo + r / G, h = r % G;
    const size_t orow = ((size_t)(t0 + pl) * hq_all + kvh * G + h) * D;
    const float inv = 1.f / l_run[n];
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) store4<T>(a.out, orow + dt * 16 + g * 4, o[n][dt], inv);
  }
}

template <typename T, int D, int G>
int launch_prefill(PrefillArgs a, int n_seqs, int max_chunk, hipStream_t st) {
  using S = PfShape<T, D, G>;
  a.n_qt = (max_chunk + S::MP - 1) / S::MP;
  a.n_work = a.n_qt * a.hkv * n_seqs;
  const int grid = (a.n_work + 7) / 8 * 8;           // whole XCD rounds
  hipLaunchKernelGGL((prefill_attention_kernel<T, D, G>), dim3(grid), dim3(kPfThreads), 0, st, a);
  return launch_status();
}

template <typename T, int D>
int prefill_g(const PrefillArgs& a, int G, int n, int mc, hipStream_t st) {
  switch (G) {
    case 1: return launch_prefill<T, D, 1>(a, n, mc, st);
    case 2: return launch_prefill<T, D, 2>(a, n, mc, st);
    case 4: return launch_prefill<T, D, 4>(a, n, mc, st);
    case 8: return launch_prefill<T, D, 8>(a, n, mc, st);
  }
  return KVC_ERR_UNSUPPORTED;
}

int dispatch_prefill(const PrefillArgs& a, int dtype, int D, int G, int n, int mc, hipStream_t st) {
  if (dtype == KVC_F32) {
    switch (D) {
      case 16: return prefill_g<float, 16>(a, G, n, mc, st);
      case 32: return prefill_g<float, 32>(a, G, n, mc, st);
      case 64: return prefill_g<float, 64>(a, G, n, mc, st);
      case 128: return prefill_g<float, 128>(a, G, n, mc, st);
    }
  } else {
    switch (D) {
      case 32: return prefill_g<bf16_tag, 32>(a, G, n, mc, st);
      case 64: return prefill_g<bf16_tag, 64>(a, G, n, mc, st);
      case 128: return prefill_g<bf16_tag, 128>(a, G, n, mc, st);
    }
  }
  return KVC_ERR_UNSUPPORTED;
}

}  // namespace kvc

extern "C" int kvc_chunked_prefill_attention(const kvc_cache* cache, const void* q, const void* k,
                                             const void* v, int32_t n_seqs, const int32_t* cu_chunk_lens,
                                             const int32_t* prefix_lens, int32_t total_tokens,
                                             int32_t max_chunk_len, const int32_t* block_table,
                                             int32_t max_blocks, int32_t Hq, float softmax_scale,
                                             void* out, void* stream) {
  int st = kvc::check_cache(cache);
  if (st != KVC_OK) return st;
  if (n_seqs < 0 || total_tokens < 0 || max_chunk_len < 0 || max_blocks < 0 || Hq <= 0)
    return KVC_ERR_SHAPE;
  if (Hq % cache->num_kv_heads != 0) return KVC_ERR_SHAPE;
  const int G = Hq / cache->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVC_ERR_UNSUPPORTED;
  if (n_seqs == 0 || total_tokens == 0 || max_chunk_len == 0) return KVC_OK;
  if (cache->num_blocks < 1) return KVC_ERR_SHAPE;   // a chunk needs somewhere to go
  if (!q || !k || !v || !cu_chunk_lens || !prefix_lens || !block_table || !out) return KVC_ERR_NULL;
  hipStream_t s = kvc::as_stream(stream);
  st = kvc::launch_chunk_append(cache, k, v, n_seqs, cu_chunk_lens, prefix_lens, total_tokens,
                                max_chunk_len, block_table, max_blocks, s);
  if (st != KVC_OK) return st;
  kvc::PrefillArgs a;
  a.q = q;
  a.kc = cache->k_cache;
  a.vc = cache->v_cache;
  a.cu = cu_chunk_lens;
  a.prefix = prefix_lens;
  a.bt = block_table;
  a.out = out;
  a.err = cache->err_flag;
  a.hkv = cache->num_kv_heads;
  a.num_blocks = cache->num_blocks;
  a.max_blocks = max_blocks;
  a.total = total_tokens;
  a.max_chunk = max_chunk_len;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  return kvc::dispatch_prefill(a, cache->dtype, cache->head_dim, G, n_seqs, max_chunk_len, s);
}
