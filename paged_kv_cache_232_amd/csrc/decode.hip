// Paged decode attention: one query token per sequence against its block-table-indexed KV cache.
//
// What is computed (vLLM-derived paged_attn.py page, PagedAttention._forward_decode_pytorch and
// forward_decode): out[b, h] = softmax(scale * q[b, h] . K^T) V over the sequence's tokens, with
// a running max / exp-sum / rescaled output carried across tiles, and (split-KV, the page's V2
// path) 512-token partitions whose statistics a second kernel merges by log-sum-exp.
//
// MI355X design. Decode moves every K/V byte exactly once, so the kernel is an HBM stream:
//   * a wave streams 32-token chunks (two 16-token half pages) of one (sequence, kv head, group
//     of <= 16 q heads) with the next chunk's loads already in flight while one is processed;
//     split-KV: one single-wave work-group per partition; direct: 4 waves per sequence take
//     chunks round robin and are combined through LDS at the end;
//   * QK^T on a 16x16x32 bf16 MFMA with the K half page as the A operand (rows = 16 tokens) and
//     the GQA group's q rows as B (16 columns); a K half page is read in contiguous wave loads
//     (1 KiB of bf16, 512 bytes of fp8 codes) and staged through the wave's LDS tile (which V
//     then reuses), fp8 codes converted to bf16 as they are read back;
//   * the score tile lands in the layout the PV MFMA needs for its B operand: each lane already
//     holds 8 probabilities of one head, so P never moves between lanes;
//   * V is read from HBM in contiguous 1 KiB wave loads, staged row-major in a per-wave LDS tile
//     (row pad chosen so transpose reads hit distinct banks) and read back with the gfx950
//     transpose read (ds_read_b64_tr_b16) as V^T, the PV MFMA's A operand;
//   * softmax runs in the log2 domain with the scale folded into one FMA before v_exp_f32; the
//     running max is raised only when it grows by more than 2^8 (a wave-uniform branch);
//   * block ids come from a per-wave table window read with v_readlane, so forming an address
//     never waits on a table load queued behind in-flight data;
//   * slots past the sequence length are masked by selection (their bits may be NaN).
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pkv {

constexpr int kDirectWaves = 4;  // waves per work-group on the direct path (split: one wave)
constexpr float kRescaleLog2 = 8.0f;  // raise a running max only when exceeded by more than this
constexpr int kPrefetch = 2;          // 32-token chunks per wave in flight (loads issued ahead)
constexpr int kMergeUnroll = 8;       // merge: partial rows per thread in flight
constexpr int kMaxStageBytes = 68 * 1024;  // split: LDS for parked partials per wave
// fp8 caches: most consecutive partitions one split wave streams (4 and 16 measured slower)
constexpr int kFp8MaxPpw = 2;

template <int D>
struct DecodeCfg {
  static constexpr int KK = D / 32;           // 32-wide d slices of the QK MFMA
  static constexpr int MT = D / 16;           // 16-row d tiles of the PV MFMA
  static constexpr int VU = D / 32;           // 16-byte V units per lane per half page
  static constexpr int RS = 2 * D + 32;       // LDS bytes per staged V row (pad: conflict-free tr reads)
  static constexpr int RSK = 2 * D + 16;      // LDS bytes per staged K row (pad: conflict-free reads)
  static constexpr int RSK8 = D + 8;          // the same for a row of fp8 K codes
  static constexpr int WAVE_LDS = 32 * RS;    // one wave's 32-row V tile
  static_assert(WAVE_LDS >= D * 16 * 4, "combine buffer must fit in a wave's V tile");
};

// One 32-token chunk in registers: per half page, each lane's K operand pieces and V pieces, 8
// elements each (16 bytes of bf16, or 8 bytes of fp8 codes).
template <int D, bool FP8>
struct DecodeChunk {
  using Piece = std::conditional_t<FP8, u32x2, u32x4>;
  Piece k[2][DecodeCfg<D>::KK];
  Piece v[2][DecodeCfg<D>::VU];
};

// 8 elements of a chunk piece as bf16 (fp8 e4m3 codes convert exactly)
__device__ __forceinline__ u32x4 piece_bf16(u32x4 x) { return x; }
__device__ __forceinline__ u32x4 piece_bf16(u32x2 x) { return fp8x8_to_bf16x8(x); }
// Non-temporal loads: every K and V load instruction reads whole 128-byte lines (a contiguous
// 1 KiB of bf16, or 512 bytes of fp8 codes, per wave) that nothing reads again. Keeping these
// lines out of the caches' normal replacement measured 8-15 % faster on the decode workloads.
__device__ __forceinline__ u32x4 load_piece_nt(const uint16_t* p, u32x4*) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 load_piece_nt(const uint8_t* p, u32x2*) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}


// scale_log2 > 0 always: the host folds a negative scale into negate_q (an exact sign flip of q)
// and replaces a zero scale by the smallest normal float (every probability is then exactly 1).
template <int D, int NW, bool SPLIT, bool FP8>
__global__ void __launch_bounds__(NW * kWave, D <= 128 ? 2 : 1)
decode_kernel(const uint16_t* __restrict__ q, const std::conditional_t<FP8, uint8_t, uint16_t>* __restrict__ kc,
              const std::conditional_t<FP8, uint8_t, uint16_t>* __restrict__ vc,
              const int32_t* __restrict__ tables,
              const int32_t* __restrict__ lens, uint16_t* __restrict__ out,
              float* __restrict__ lse, float* __restrict__ o_part, float* __restrict__ m_part,
              float* __restrict__ l_part, int Hq, int Hkv, int G, int n_hg, int BS, int NB,
              int max_blocks, int PT, int Pmax, float scale_log2, float v_scale, int negate_q,
              int bs_shift, int window, int pair_order, int ppw) {
  using C = DecodeCfg<D>;
  using Chunk = DecodeChunk<D, FP8>;
  using KVT = std::conditional_t<FP8, uint8_t, uint16_t>;
  using Piece = typename Chunk::Piece;
  __shared__ __attribute__((aligned(16))) char smem[NW * C::WAVE_LDS];
  __shared__ float sm_m[NW][16];
  // split with several partitions per wave: the finished partitions' normalised partials wait in
  // dynamic LDS until the wave has stopped streaming (a global store among loads in flight would
  // make every later wait drain them all)
  extern __shared__ __attribute__((aligned(16))) float stage[];
  __shared__ float sm_l[NW][16];

  const int p = blockIdx.x;
  const int kh = blockIdx.y / n_hg;
  const int hg = blockIdx.y - kh * n_hg;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, kept scalar
  const int col = lane & 15;  // head column of the MFMA tiles
  const int qg = lane >> 4;   // lane group 0..3
  int b = blockIdx.z;
  if (pair_order) {
    // Direct path, batch <= 64: work-group z takes the sequence of length rank z for z < B/2 and
    // of rank B-1-(z-B/2) after, so the two work-groups the dispatcher places on one CU (z and
    // z + B/2) pair a long sequence with a short one. Ties rank by index.
    const int B = gridDim.z;
    const int h = (B + 1) / 2;
    const int target = (int)blockIdx.z < h ? (int)blockIdx.z : B - 1 - ((int)blockIdx.z - h);
    int mine = -1;
    if (lane < B) mine = clampi(lens[lane], 0, max_blocks * BS);
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int lj = __builtin_amdgcn_readlane(mine, j);
      rank += (lj > mine || (lj == mine && j < lane)) ? 1 : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && rank == target);
    b = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
  }

  int L = clampi(lens[b], 0, max_blocks * BS);
  if (SPLIT && window == 0) L = min(L, Pmax * PT);
  // sliding window: keys [t_lo, L); chunks stay 32-token aligned, keys before t_lo are masked
  const int t_lo = window > 0 ? max(0, L - window) : 0;
  // windowed split: grid x and the partials count partitions from the one holding t_lo
  const int p_base = (SPLIT && window > 0) ? t_lo / PT : 0;
  int t_begin = t_lo & ~31, t_end = L;
  if constexpr (SPLIT) {
    // partitions p_base + p*ppw .. + ppw - 1, streamed by one wave
    const int pa = p_base + p * ppw;
    t_begin = max(pa * PT, t_begin);
    t_end = min(L, (pa + ppw) * PT);
    if (t_begin >= t_end) return;  // uniform over the work-group (no partial is written)
  }
  const int p_first = SPLIT ? t_begin / PT : 0;  // partition of the first chunk
  int next_boundary = SPLIT ? (p_first + 1) * PT : 0;

  const int gcol = hg * 16 + col;
  const bool col_ok = gcol < G;
  // staged partial slot: the group's valid head columns x (D + 4) floats, then m and l per column
  const int n_valid = min(16, G - hg * 16);
  const int slot_floats = n_valid * (D + 4) + 32;
  const int hq = kh * G + min(gcol, G - 1);

  // B operand of QK: q[hq][kk*32 + 8*qg .. +8]
  bf16x8 qreg[C::KK];
  {
    const uint16_t* qp = q + ((size_t)b * Hq + hq) * D + 8 * qg;
    const uint32_t flip = negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      u32x4 v = load16(qp + kk * 32);
      v ^= u32x4{flip, flip, flip, flip};
      if (!col_ok) v = u32x4{0, 0, 0, 0};
      qreg[kk] = as_bf16x8(v);
    }
  }

  f32x4 o[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // log2 units
  float l_run = 0.f;

  char* vbuf = smem + w * C::WAVE_LDS;
  const uint16_t* vl = reinterpret_cast<const uint16_t*>(vbuf);
  const int n_chunks = (t_end - t_begin + 31) >> 5;
  const int32_t* trow = tables + (size_t)b * max_blocks;
  const size_t head_stride = (size_t)BS * D;
  const size_t block_stride = (size_t)Hkv * head_stride;
  const int last = t_end - 1;
  // transpose-read address of the V^T operand: group qg reads token rows 4*qg + (l%16)/4
  // (+16 for the second half page) at columns 4*(l%4) of each 16-wide d tile
  const int tr_off = (4 * qg + ((lane & 15) >> 2)) * (C::RS / 2) + 4 * (lane & 3);

  TableWindow tw;
  tw.init(trow, max_blocks, (t_begin + w * 32) >> bs_shift, lane);

  const int voff = lane * 8;          // this lane's first V element within a half page

  auto load = [&](Chunk& ch, int c) {
    const int cs = t_begin + c * 32;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int tok0 = cs + 16 * hh;
      const int tk = tok0 < t_end ? tok0 : cs;  // an all-masked half page re-reads a valid one
      const int blk = clampi(tw.get(tk >> bs_shift, lane), 0, NB - 1);
      const size_t base = (size_t)blk * block_stride + (size_t)kh * head_stride +
                          (size_t)(tk & (BS - 1)) * D;
      const KVT* kp = kc + base;
      const KVT* vp = vc + base;
#pragma unroll
      for (int i = 0; i < C::KK; ++i) {
        // whole rows like V, contiguous per instruction (1 KiB bf16, 512 bytes fp8), staged
        // through LDS below
        ch.k[hh][i] = load_piece_nt(kp + voff + i * 512, (Piece*)nullptr);
      }
#pragma unroll
      for (int i = 0; i < C::VU; ++i) ch.v[hh][i] = load_piece_nt(vp + voff + i * 512, (Piece*)nullptr);
    }
  };

  auto process = [&](const Chunk& ch, int c) {
    const int cs = t_begin + c * 32;
    // only a partition's last chunk holds slack rows, only a window's first one keys before t_lo
    const bool partial = cs + 31 > last || cs < t_lo;
    // S^T[token][head] for the two half pages
    f32x4 s[2];
    if constexpr (FP8) {
      // fp8 K rows staged in the wave's LDS tile (row stride RSK8 bytes), read back as 8-code
      // operand pieces and converted to bf16; the V rows then overwrite the tile
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < C::KK; ++i) {
          const int u = i * 64 + lane;
          const int row = u / (D / 8);
          *reinterpret_cast<u32x2*>(vbuf + (16 * hh + row) * C::RSK8 + (u - row * (D / 8)) * 8) = ch.k[hh][i];
        }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        s[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk)
          s[hh] = mfma16(as_bf16x8(fp8x8_to_bf16x8(*reinterpret_cast<const u32x2*>(
                             vbuf + (16 * hh + col) * C::RSK8 + 32 * kk + 8 * qg))),
                         qreg[kk], s[hh]);
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      // K rows staged in the wave's LDS tile (row stride RSK), read back as the A operand; the V
      // rows then overwrite the tile (LDS operations of one wave run in order)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < C::KK; ++i) {
          const int u = i * 64 + lane;
          const int row = u / (D / 8);
          *reinterpret_cast<u32x4*>(vbuf + (16 * hh + row) * C::RSK + (u - row * (D / 8)) * 16) = ch.k[hh][i];
        }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        s[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk)
          s[hh] = mfma16(as_bf16x8(*reinterpret_cast<const u32x4*>(
                             vbuf + (16 * hh + col) * C::RSK + (32 * kk + 8 * qg) * 2)),
                         qreg[kk], s[hh]);
      }
      __builtin_amdgcn_wave_barrier();
    }
    // stage V rows in LDS; rows past the end are zeroed (select, so NaN slack never leaks)
    if (!partial) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < C::VU; ++i) {
          const int u = i * 64 + lane;
          const int row = u / (D / 8);
          *reinterpret_cast<u32x4*>(vbuf + (16 * hh + row) * C::RS + (u - row * (D / 8)) * 16) = piece_bf16(ch.v[hh][i]);
        }
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < C::VU; ++i) {
          const int u = i * 64 + lane;
          const int row = u / (D / 8);
          u32x4 val = piece_bf16(ch.v[hh][i]);
          const int tok = cs + 16 * hh + row;
          if (tok > last || tok < t_lo) val = u32x4{0, 0, 0, 0};
          *reinterpret_cast<u32x4*>(vbuf + (16 * hh + row) * C::RS + (u - row * (D / 8)) * 16) = val;
        }
    }
    // raw scores (masked past the end on a partial chunk); running max in log2 units, raised lazily
    float sv[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[hh * 4 + r] = s[hh][r];
    if (partial) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tok = cs + 16 * (j >> 2) + 4 * qg + (j & 3);
        if (tok > last || tok < t_lo) sv[j] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mx = max_xor32(max_xor16(mx));
    const float tmax = mx * scale_log2;
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescaleLog2) != 0) {
      const float m_new = fmaxf(m_run, tmax);
      const float corr = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) o[mt] *= corr;
    }
    const float neg_m = -m_run;  // finite: every chunk holds at least one valid token
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = fast_exp2(__builtin_fmaf(sv[j], scale_log2, neg_m));
      l_run += pv[j];
    }
    // B operand of PV: k-index 8*qg + j <-> token 16*(j/4) + 4*qg + j%4, exactly this lane's scores
    const bf16x8 pb = pack_bf16x8(pv);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      const uint16_t* vp = vl + tr_off + mt * 16;
      const u32x2 lo = lds_read_tr16(vp);
      const u32x2 hi = lds_read_tr16(vp + 16 * (C::RS / 2));
      o[mt] = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb, o[mt]);
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (SPLIT && NW == 1) {
      if (cs + 32 == next_boundary && next_boundary < t_end) {
        // a partition is complete: park its partial, start the next one afresh
        const float lt = sum_xor32(sum_xor16(l_run));
        const float inv = lt > 0.f ? v_scale / lt : 0.f;
        float* sl = stage + (next_boundary / PT - 1 - p_first) * slot_floats;
        if (col_ok) {
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt)
            *reinterpret_cast<f32x4*>(sl + col * (D + 4) + mt * 16 + 4 * qg) = o[mt] * inv;
          if (qg == 0) {
            sl[n_valid * (D + 4) + col] = m_run;
            sl[n_valid * (D + 4) + 16 + col] = lt;
          }
        }
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
        next_boundary += PT;
      }
    }
  };

  // chunks w, w+NW, ... with the next PF-1 chunks' loads in flight while one is processed.
  // The steady-state loop issues its look-ahead loads unconditionally, so the compiler can count
  // exactly which loads a chunk must wait for; the tail drains in a guarded epilogue.
  {
    constexpr int PF = kPrefetch;
    Chunk ring[PF];
    int c = w;
#pragma unroll
    for (int i = 0; i < PF - 1; ++i)
      if (c + i * NW < n_chunks) load(ring[i], c + i * NW);
    while (c + (2 * PF - 2) * NW < n_chunks) {
#pragma unroll
      for (int sl = 0; sl < PF; ++sl) {
        load(ring[(sl + PF - 1) % PF], c + (PF - 1) * NW);
        process(ring[sl], c);
        c += NW;
      }
    }
#pragma unroll
    for (int sl = 0; sl < 2 * PF - 1; ++sl) {
      if (c < n_chunks) {
        const int ahead = c + (PF - 1) * NW;
        if (ahead < n_chunks) load(ring[(sl + PF - 1) % PF], ahead);
        process(ring[sl % PF], c);
        c += NW;
      }
    }
  }

  // lane-group partial sums -> per-column sums (m_run is already uniform per column)
  l_run = sum_xor32(sum_xor16(l_run));

  if constexpr (NW == 1) {
    // a single wave owns the whole work item: normalise and write straight from registers
    if (!col_ok) return;
    const int hout = kh * G + gcol;
    const float inv = l_run > 0.f ? v_scale / l_run : 0.f;
    if constexpr (SPLIT) {
      const int p_last = (t_end - 1) / PT;
      const size_t pi = ((size_t)b * Pmax + (p_last - p_base)) * Hq + hout;
      float* op = o_part + pi * D + 4 * qg;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) *reinterpret_cast<f32x4*>(op + mt * 16) = o[mt] * inv;
      if (qg == 0) {
        m_part[pi] = m_run;
        l_part[pi] = l_run;
      }
      // the parked partitions p_first .. p_last - 1
      for (int pp = p_first; pp < p_last; ++pp) {
        const float* sl = stage + (pp - p_first) * slot_floats;
        const size_t pj = ((size_t)b * Pmax + (pp - p_base)) * Hq + hout;
        float* fp = o_part + pj * D + 4 * qg;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
          *reinterpret_cast<f32x4*>(fp + mt * 16) =
              *reinterpret_cast<const f32x4*>(sl + col * (D + 4) + mt * 16 + 4 * qg);
        if (qg == 0) {
          m_part[pj] = sl[n_valid * (D + 4) + col];
          l_part[pj] = sl[n_valid * (D + 4) + 16 + col];
        }
      }
    } else {
      uint16_t* op = out + ((size_t)b * Hq + hout) * D + 4 * qg;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
        *reinterpret_cast<u32x2*>(op + mt * 16) =
            u32x2{pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv), pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv)};
      if (lse != nullptr && qg == 0)
        lse[(size_t)b * Hq + hout] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
    }
    return;
  } else {
    __syncthreads();  // every wave is done with its V tile; reuse it for O^T [d][16]
    float* obuf = reinterpret_cast<float*>(vbuf);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) obuf[(mt * 16 + 4 * qg + r) * 16 + col] = o[mt][r];
    if (lane < 16) {
      sm_m[w][lane] = m_run;
      sm_l[w][lane] = l_run;
    }
    __syncthreads();

    constexpr int TPC = NW * kWave / 16;  // threads per head column
    constexpr int DPT = D / TPC;          // outputs per thread
    const int t = threadIdx.x;
    const int oc = t / TPC;
    const int dpart = t - oc * TPC;
    if (hg * 16 + oc >= G) return;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, sm_m[w2][oc]);
    float f[NW];
    float lsum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const float mw = sm_m[w2][oc];
      f[w2] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      lsum += f[w2] * sm_l[w2][oc];
    }
    const float inv = lsum > 0.f ? v_scale / lsum : 0.f;
    float acc[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const int d = dpart * DPT + i;
      float a = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2)
        a += f[w2] * reinterpret_cast<const float*>(smem + w2 * C::WAVE_LDS)[d * 16 + oc];
      acc[i] = a * inv;
    }
    const int hout = kh * G + hg * 16 + oc;
    static_assert(!SPLIT, "split partitions run single-wave work-groups");
    if (o_part != nullptr) {
      // streamed attention: fold this launch's (max, exp-sum, normalised output) into the running
      // state of (b, hout). The column's threads are one wave: every lane reads before any writes.
      const size_t si = (size_t)b * Hq + hout;
      const float ms = m_part[si];
      const float ls = l_part[si];
      const float Mn = fmaxf(ms, M);
      const float ws = (ms == -INFINITY) ? 0.f : ls * fast_exp2(ms - Mn);
      const float wp = (M == -INFINITY) ? 0.f : lsum * fast_exp2(M - Mn);
      const float tot = ws + wp;
      const float as = tot > 0.f ? ws / tot : 0.f;
      const float ap = tot > 0.f ? wp / tot : 0.f;
      float* op = o_part + si * D + dpart * DPT;
#pragma unroll
      for (int i = 0; i < DPT; i += 4) {
        const f32x4 old = *reinterpret_cast<const f32x4*>(op + i);
        *reinterpret_cast<f32x4*>(op + i) =
            old * as + f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]} * ap;
      }
      if (dpart == 0) {
        m_part[si] = tot > 0.f ? Mn : -INFINITY;
        l_part[si] = tot;
      }
    } else {
      uint16_t* op = out + ((size_t)b * Hq + hout) * D + dpart * DPT;
#pragma unroll
      for (int i = 0; i < DPT; i += 4)
        *reinterpret_cast<u32x2*>(op + i) =
            u32x2{pack_bf16x2(acc[i], acc[i + 1]), pack_bf16x2(acc[i + 2], acc[i + 3])};
      if (lse != nullptr && dpart == 0)
        lse[(size_t)b * Hq + hout] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
    }
  }
}

// Streamed attention state [B, Hq]: normalised output rows o (fp32, D), running max m (log2 units)
// and exp-sum l. begin: o = 0, m = -inf, l = 0 (a fill kernel, safe inside a captured graph).
__global__ void __launch_bounds__(256)
stream_state_begin_kernel(float* __restrict__ o, float* __restrict__ m, float* __restrict__ l,
                          int64_t rows, int D) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * D; i += stride) {
    o[i] = 0.f;
    if (i < rows) {
      m[i] = -INFINITY;
      l[i] = 0.f;
    }
  }
}

// finalize: out = bf16(o) (already normalised; zero rows for an empty state), lse in natural log
__global__ void __launch_bounds__(256)
stream_state_finalize_kernel(const float* __restrict__ o, const float* __restrict__ m,
                             const float* __restrict__ l, uint16_t* __restrict__ out,
                             float* __restrict__ lse, int64_t rows, int D) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * D / 2; i += stride) {
    const float2 v = reinterpret_cast<const float2*>(o)[i];
    reinterpret_cast<uint32_t*>(out)[i] = pack_bf16x2(v.x, v.y);
    if (lse != nullptr && i < rows) lse[i] = l[i] > 0.f ? (m[i] + __log2f(l[i])) * kLn2 : -INFINITY;
  }
}

// Log-sum-exp merge of split partials: one work-group per (q head, sequence). Thread group g
// (U threads, one float4 of the row each) folds partitions g, g+NG, ... into a running
// (max, exp-sum, weighted output), loading kMergeUnroll partitions at a time; the NG group states
// are then combined through LDS. One pass over the partials, all of a batch's loads in flight.
template <int D, int NT>
__global__ void __launch_bounds__(NT)
decode_merge_kernel(const float* __restrict__ o_part, const float* __restrict__ m_part,
                    const float* __restrict__ l_part, const int32_t* __restrict__ lens,
                    uint16_t* __restrict__ out, float* __restrict__ lse, int Hq, int max_blocks,
                    int BS, int PT, int Pmax, int window) {
  constexpr int U = D / 4;    // float4 units per partial row
  constexpr int NG = NT / U;  // partition groups
  __shared__ float sm[NG];
  __shared__ float sl[NG];
  __shared__ f32x4 so[NG][U];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  int L = clampi(lens[b], 0, max_blocks * BS);
  if (window == 0) L = min(L, Pmax * PT);
  // a sliding window's partials start at the partition holding its first key
  const int p_lo = window > 0 ? max(0, L - window) / PT : 0;
  const int P = min((L + PT - 1) / PT, p_lo + Pmax);  // partitions holding tokens (finite max each)
  // partial p of (b, h) is row (b * Pmax + p - p_lo) * Hq + h
  const size_t pi0 = (size_t)b * Pmax * Hq + h;
  const int u = t % U;
  const int g = t / U;

  float Mg = -INFINITY;  // log2 units
  float Sg = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = p_lo + g; p0 < P; p0 += NG * kMergeUnroll) {
    f32x4 x[kMergeUnroll];
    float mp[kMergeUnroll], lp[kMergeUnroll];
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j) {
      const int p = p0 + j * NG;
      x[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      mp[j] = -INFINITY;
      lp[j] = 0.f;
      if (p < P) {
        const size_t pi = pi0 + (size_t)(p - p_lo) * Hq;
        x[j] = reinterpret_cast<const f32x4*>(o_part + pi * D)[u];
        mp[j] = m_part[pi];
        lp[j] = l_part[pi];
      }
    }
    float Mb = Mg;
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j) Mb = fmaxf(Mb, mp[j]);
    const float c = (Mg == -INFINITY) ? 0.f : fast_exp2(Mg - Mb);
    acc *= c;
    Sg *= c;
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j) {
      const float wj = (mp[j] == -INFINITY) ? 0.f : lp[j] * fast_exp2(mp[j] - Mb);
      Sg += wj;
      acc += wj * x[j];
    }
    Mg = Mb;
  }
  if (u == 0) {
    sm[g] = Mg;
    sl[g] = Sg;
  }
  so[g][u] = acc;
  __syncthreads();
  if (g != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) M = fmaxf(M, sm[gg]);
  float S = 0.f;
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    const float c = (sm[gg] == -INFINITY) ? 0.f : fast_exp2(sm[gg] - M);
    S += c * sl[gg];
    sum += c * so[gg][u];
  }
  const float inv = S > 0.f ? 1.f / S : 0.f;
  sum *= inv;
  *reinterpret_cast<u32x2*>(out + ((size_t)b * Hq + h) * D + u * 4) =
      u32x2{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
  if (lse != nullptr && u == 0)
    lse[(size_t)b * Hq + h] = S > 0.f ? (M + __log2f(S)) * kLn2 : -INFINITY;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int decode_max_ppw(int num_q_heads, int num_kv_heads, int head_dim) {
  const int G = num_q_heads / num_kv_heads;
  const int slot_bytes = (std::min(16, G) * (head_dim + 4) + 32) * (int)sizeof(float);
  return std::min(16, 1 + kMaxStageBytes / slot_bytes);
}

DecodeWorkspaceLayout decode_workspace_layout(int batch, int num_q_heads, int head_dim,
                                              int max_seq_len, int partition_tokens) {
  if (partition_tokens <= 0) return DecodeWorkspaceLayout{0, 0, 0, 0, 0};
  const int P = max_seq_len > 0 ? (max_seq_len + partition_tokens - 1) / partition_tokens : 1;
  return decode_workspace_layout_p(batch, num_q_heads, head_dim, P);
}

int decode_window_partitions(int max_seq_len, int window, int partition_tokens) {
  const int all = max_seq_len > 0 ? (max_seq_len + partition_tokens - 1) / partition_tokens : 1;
  // keys [L - window, L) touch at most ceil(window / PT) + 1 partitions
  const long span = ((long)window + partition_tokens - 1) / partition_tokens + 1;
  return (int)std::min<long>(all, span);
}

DecodeWorkspaceLayout decode_workspace_layout_p(int batch, int num_q_heads, int head_dim, int P) {
  DecodeWorkspaceLayout w{0, 0, 0, 0, 0};
  const size_t rows = (size_t)batch * num_q_heads * P;
  w.max_partitions = P;
  w.o_off = 0;
  w.m_off = align256(rows * head_dim * sizeof(float));
  w.l_off = w.m_off + align256(rows * sizeof(float));
  w.total = w.l_off + align256(rows * sizeof(float));
  return w;
}

template <int D, bool FP8>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  using KVT = std::conditional_t<FP8, uint8_t, uint16_t>;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int n_hg = (G + 15) / 16;
  // fp8 cache: scores are q . code * (scale * k_scale), outputs sum p * code * v_scale
  const float k_scale = FP8 ? a.k_scale : 1.f;
  const float v_scale = FP8 ? a.v_scale : 1.f;
  float scale_log2 = a.scale * k_scale * kLog2e;
  const int negate_q = scale_log2 < 0.f;
  if (negate_q) scale_log2 = -scale_log2;
  if (!(scale_log2 >= 1.17549435e-38f)) scale_log2 = 1.17549435e-38f;  // zero (or denormal) scale
  const int bs_shift = __builtin_ctz((unsigned)a.block_size);
  if (a.partition_tokens > 0) {
    // Long contexts: a wave streams up to 16 consecutive partitions (fewer, longer streams run
    // faster), parking all but the last partial in LDS; the largest count that the LDS budget
    // allows and that still leaves 512 waves (two per CU) is taken.
    const int slot_bytes = (std::min(16, G) * (D + 4) + 32) * (int)sizeof(float);
    const int lds_cap = decode_max_ppw(a.num_q_heads, a.num_kv_heads, D);
    // Partitions holding visible keys: with a sliding window only the last ones. The fp8 cache
    // streams at most two partitions per wave (measured fastest there: four or more were slower).
    int p_act = a.max_partitions;
    if (a.window > 0) p_act = std::min(p_act, (a.window + 31) / a.partition_tokens + 2);
    int ppw = 1;
    if (a.ppw_override > 0) {
      ppw = std::min(a.ppw_override, lds_cap);
    } else if (p_act >= 64) {
      const long units = (long)a.batch * a.num_kv_heads * n_hg;
      for (int c = FP8 ? kFp8MaxPpw : 16; c > 1; c /= 2)
        if (c <= lds_cap && units * ((p_act + c - 1) / c) >= 512) {
          ppw = c;
          break;
        }
    }
    const size_t stage_bytes = (size_t)(ppw - 1) * slot_bytes;
    const dim3 grid((a.max_partitions + ppw - 1) / ppw, a.num_kv_heads * n_hg, a.batch);
    hipLaunchKernelGGL((decode_kernel<D, 1, true, FP8>), grid, dim3(kWave), stage_bytes, stream,
                       (const uint16_t*)a.q, (const KVT*)a.k_cache, (const KVT*)a.v_cache,
                       a.block_tables, a.seq_lens, (uint16_t*)a.out, a.lse, a.o_part, a.m_part,
                       a.l_part, a.num_q_heads, a.num_kv_heads, G, n_hg, a.block_size,
                       a.num_blocks, a.max_blocks_per_seq, a.partition_tokens, a.max_partitions,
                       scale_log2, v_scale, negate_q, bs_shift, a.window, 0, ppw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // long splits take 1024 threads per (head, sequence), so one batch of loads covers them
    const dim3 mgrid(a.num_q_heads, a.batch);
    if (a.max_partitions > 4 * kMergeUnroll)
      hipLaunchKernelGGL((decode_merge_kernel<D, 1024>), mgrid, dim3(1024), 0, stream, a.o_part,
                         a.m_part, a.l_part, a.seq_lens, (uint16_t*)a.out, a.lse, a.num_q_heads,
                         a.max_blocks_per_seq, a.block_size, a.partition_tokens, a.max_partitions,
                         a.window);
    else
      hipLaunchKernelGGL((decode_merge_kernel<D, 256>), mgrid, dim3(256), 0, stream, a.o_part,
                         a.m_part, a.l_part, a.seq_lens, (uint16_t*)a.out, a.lse, a.num_q_heads,
                         a.max_blocks_per_seq, a.block_size, a.partition_tokens, a.max_partitions,
                         a.window);
    return hipGetLastError();
  }
  // direct path; with a stream state (o_part etc. set, no partitions) the result is folded into it
  const dim3 grid(1, a.num_kv_heads * n_hg, a.batch);
  hipLaunchKernelGGL((decode_kernel<D, kDirectWaves, false, FP8>), grid, dim3(kDirectWaves * kWave),
                     0, stream, (const uint16_t*)a.q, (const KVT*)a.k_cache, (const KVT*)a.v_cache,
                     a.block_tables, a.seq_lens, (uint16_t*)a.out, a.lse, a.o_part, a.m_part,
                     a.l_part, a.num_q_heads, a.num_kv_heads, G, n_hg, a.block_size, a.num_blocks,
                     a.max_blocks_per_seq, 0, 1, scale_log2, v_scale, negate_q, bs_shift, a.window,
                     (a.batch <= 64 && a.o_part == nullptr) ? 1 : 0, 1);
  return hipGetLastError();
}

template <bool FP8>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_decode_d<64, FP8>(a, stream);
    case 128: return launch_decode_d<128, FP8>(a, stream);
    case 256: return launch_decode_d<256, FP8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_state_begin(float* o, float* m, float* l, int rows, int head_dim,
                                     hipStream_t stream) {
  const int64_t n = (int64_t)rows * head_dim;
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(stream_state_begin_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, o, m, l,
                     (int64_t)rows, head_dim);
  return hipGetLastError();
}

hipError_t launch_stream_state_finalize(const float* o, const float* m, const float* l, void* out,
                                        float* lse, int rows, int head_dim, hipStream_t stream) {
  const int64_t n = (int64_t)rows * head_dim / 2;
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(stream_state_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, o, m,
                     l, (uint16_t*)out, lse, (int64_t)rows, head_dim);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.kv_fp8 ? launch_decode_t<true>(a, stream) : launch_decode_t<false>(a, stream);
}

}  // namespace pkv
