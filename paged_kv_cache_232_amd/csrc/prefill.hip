// Ragged (varlen) and paged prefill attention on bf16 MFMA.
//
// What is computed: for request b, query row i (rows qo_indptr[b]..qo_indptr[b+1] of q) attends
// to its keys 0..kv_len-1 (contiguous rows kv_indptr[b].. of k/v, or cached tokens read through the
// block table); with causal masking, row i sees key j iff j <= i + (kv_len - qo_len). Sources: the
// spark_runtime/flashinfer.rs page (ragged_prefill_bf16_hd256 and its CPU-reference test) and the
// vLLM-derived paged_attn.py page (_forward_prefix_pytorch: cached prefix unmasked, chunk causal).
//
// MI355X design (a dense contraction, so MFMA-bound):
//   * head_dim <= 128: work-group = 4 waves x 32 rows over hp q heads of one kv head
//     (hp = gcd(G, 4)), a tile of 128 / hp rows; head_dim 256: 12 waves x 16 rows over
//     hp = gcd(G, 12) heads, a tile of 192 / hp rows. The heads of a work-group share each staged
//     K / V tile, and all its waves see the same causal extent;
//   * head_dim <= 128: K and V tiles of 32 keys go straight from HBM into LDS with direct-to-LDS
//     loads (global_load_lds_dwordx4), K three tiles ahead and V one tile ahead in rings of 4 and
//     2 tiles, their 16-byte units permuted within each row so that the MFMA operand reads are
//     free of bank conflicts; one explicit wait and barrier per tile. The 32-key tiles keep a
//     wave at 166 VGPRs and a work-group at 48 KB of LDS, so three work-groups share a CU (three
//     waves per SIMD); with 64-key tiles two did, and the ragged prefill ran 3-4 % slower;
//   * head_dim 256 (16-row form below, 12 waves): tiles are loaded into registers a tile ahead and
//     staged into padded LDS rows (direct-to-LDS loads measured slower there);
//   * the QK^T MFMAs are scheduled with four LDS reads of K in flight;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the wave's Q rows held in
//     registers for the whole kernel), so each lane holds 16 keys of ONE query: the row max needs
//     one cross-lane step, and the lane's probabilities are already the B operand of
//     O^T += V^T P^T with no lane exchange;
//   * softmax in the log2 domain; causal kv tiles above the diagonal are skipped, only tiles that
//     cross the diagonal or the ragged end are masked;
//   * work-groups are mapped to XCDs so that all q heads sharing one kv head run on one XCD
//     (its L2 then serves the K/V re-reads of every head of the group);
//   * (request, q tile) work items run longest-first (most visible keys first), from a schedule
//     built on the host (passed with the launch) or, for long schedules, on the device.
#include <math.h>

#include <algorithm>
#include <type_traits>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace pkv {

// Work-group schedule: entry y of the grid's y dimension is (request << 16 | q tile), sorted by
// decreasing visible keys, so the hardware dispatcher starts the longest work first (greedy
// longest-first list scheduling). Up to kMaxOrder entries are built on the host from the length
// copies and passed by value; a longer schedule is built on the device by prefill_plan_kernel
// into the caller's workspace (entries past the device's tile count read 0xffffffff: no work).
constexpr int kMaxOrder = 768;
struct TileOrder {
  int32_t n;
  uint32_t e[kMaxOrder];
};
constexpr uint32_t kNoTile = 0xffffffffu;

constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kBM = 32 * kPrefillWaves;  // query rows per work-group
// A row's running max is only raised (and O, l rescaled) when a tile's max exceeds it by more than
// this many log2 units; otherwise probabilities are taken against the stale max and stay <= 2^8.
constexpr float kRescaleLog2 = 8.0f;
// LDS reads of K kept in flight ahead of the QK^T MFMAs (4 measured best; 2 is the default schedule)
constexpr int kQkAhead = 4;

// Work-group (x, y) -> (q head h, schedule row y). The hardware deals work-groups to the 8 XCDs
// round robin by linear id, i.e. by x % 8 when Hq % 8 == 0. With xcd_group = 8 / Hkv > 0, each
// group of xcd_group consecutive y rows holds 8 G work-groups and XCD c takes the G q heads of
// kv head c % Hkv for row y0 + c / Hkv: every q head that reads one K/V stream runs on one XCD,
// whose L2 then serves the re-reads. Else, with xcd_heads = Hq / 8 > 0, XCD c takes q heads
// c * xcd_heads .. +xcd_heads-1 of every row; else the plain mapping.
__device__ __forceinline__ void xcd_map(int Hq, int Hkv, int G, int xcd_group, int xcd_heads,
                                        int& h, int& y) {
  h = blockIdx.x;
  y = blockIdx.y;
  if (xcd_group > 0) {
    const int idg = (int)(blockIdx.y % xcd_group) * Hq + (int)blockIdx.x;
    const int c = idg & 7;
    h = (c % Hkv) * G + (idg >> 3);
    y = (int)blockIdx.y - (int)(blockIdx.y % xcd_group) + c / Hkv;
  } else if (xcd_heads > 0) {
    h = (blockIdx.x & 7) * xcd_heads + (blockIdx.x >> 3);
  }
}

// Scheduling hint for the QK^T loop of N MFMAs, each fed by one LDS read of K: keep AHEAD reads
// in flight ahead of the MFMAs (the default schedule issues them two at a time, just before use,
// so each MFMA pair waits out an LDS latency).
template <int N, int AHEAD>
__device__ __forceinline__ void sched_qk_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// One K or V tile of BN keys sits in LDS unpadded (row r at r * D elements) with its 16-byte units
// permuted within the row: logical unit c of row r is stored at unit c ^ swz(r). A direct-to-LDS
// load writes 1 KiB contiguously, so rows cannot be padded; the permutation instead spreads the
// reads below over all 64 banks: 16 consecutive rows read at one logical unit (K as the MFMA A
// operand, 16 lanes per LDS cycle) land on 16 different units, and 4 rows x 4 units of a V^T
// transpose read (32 lanes per cycle) on 16 different units. It depends on r & 15 only.
template <int UPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (UPR == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);  // 2 rows per 256 bytes
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}

template <int D>
struct PrefillCfg {
  static constexpr int BN = 32;                     // keys per kv tile
  static constexpr int KS = D / 16;                 // 16-wide d steps of QK^T
  static constexpr int MT = BN / 32;                // 32-key tiles of S^T
  static constexpr int PS = BN / 16;                // 16-key steps of PV
  static constexpr int DT = D / 32;                 // 32-wide d tiles of O^T
  static constexpr int UPR = D / 8;                 // 16-byte units per row
  static constexpr int TILE = BN * D;               // elements of one K or V tile
  static constexpr int ROWS_PER_LOAD = kWave / UPR; // rows one wave load instruction fills
  static constexpr int NL = BN * UPR / (kWave * kPrefillWaves);  // load instructions per wave per tile
  static constexpr int RSO = D + 8;                 // row stride of the staged output tile
  // K tiles in a ring of 4 (loaded three tiles ahead), V tiles in a ring of 2 (one tile ahead):
  // K is needed first in a step, so it gets the longer lead (V two tiles ahead measured slower)
  static constexpr int KBUF = 4, VBUF = 2;
  static constexpr int LDS_ELEMS =
      ((KBUF + VBUF) * TILE > kBM * RSO) ? (KBUF + VBUF) * TILE : kBM * RSO;
  static_assert(NL * kWave * kPrefillWaves == BN * UPR, "tile units must divide evenly");
  static_assert(ROWS_PER_LOAD <= 16, "a load instruction's rows must stay inside one block");
};

// The (request, q tile) a work-group runs and that request's extents, read from the device
// copies of the offsets and clamped to the buffers the host sized (q / out hold total_q rows,
// ragged k / v total_kv rows, a table row max_blocks blocks), so offsets that disagree with their
// host copies give wrong rows, never an access outside those buffers. Returns false when the
// work-group has nothing to do.
struct TileWork {
  int b, qt, q0, qo, kv;
  int64_t kv0;
};
template <bool PAGED>
__device__ __forceinline__ bool resolve_tile(int y, const TileOrder& order,
                                             const uint32_t* __restrict__ order_dev,
                                             const int32_t* __restrict__ qo_indptr,
                                             const int32_t* __restrict__ kv_indptr,
                                             const int32_t* __restrict__ kv_lens, int batch,
                                             int total_q, int total_kv, int kv_cap, int BM,
                                             TileWork& t) {
  // made explicitly wave-uniform: the request's extents then stay scalar, and so do the block-table
  // reads the tile loads address from (a vector table read would wait for every load in flight)
  // two separate reads (a select of the two pointers would make one flat load of a generic
  // address, a vector load waited on in full, in place of a scalar load)
  uint32_t sched;
  if (order_dev != nullptr) {
    sched = order_dev[y];
  } else {
    sched = order.e[min(y, kMaxOrder - 1)];
    __asm__ volatile("" : "+s"(sched));  // keeps the two reads apart
  }
  sched = (uint32_t)__builtin_amdgcn_readfirstlane((int)sched);
  if (sched == kNoTile) return false;
  t.b = (int)(sched >> 16);
  t.qt = (int)(sched & 0xffffu);
  if (t.b >= batch) return false;
  t.q0 = __builtin_amdgcn_readfirstlane(clampi(qo_indptr[t.b], 0, total_q));
  t.qo = __builtin_amdgcn_readfirstlane(clampi(qo_indptr[t.b + 1], t.q0, total_q) - t.q0);
  if constexpr (PAGED) {
    t.kv0 = 0;
    t.kv = __builtin_amdgcn_readfirstlane(clampi(kv_lens[t.b], 0, kv_cap));
  } else {
    const int k0 = __builtin_amdgcn_readfirstlane(clampi(kv_indptr[t.b], 0, total_kv));
    t.kv0 = k0;
    t.kv = __builtin_amdgcn_readfirstlane(clampi(kv_indptr[t.b + 1], k0, total_kv) - k0);
  }
  return t.qt < (t.qo + BM - 1) / BM;
}

struct RaggedLoader {
  int64_t row0;  // first kv row of the request
  int Hkv, kh, D;
  __device__ __forceinline__ size_t row_offset(int n) const {
    return ((size_t)(row0 + n) * Hkv + kh) * D;
  }
};

// Rows of one load instruction of a wave never straddle a block (at most 16 aligned rows per
// instruction, blocks are multiples of 16 rows), so the block id is wave-uniform: it is read with a
// scalar load from the request's table row. (A vector table load between the tile loads would make
// the compiler wait for every tile load in flight before forming the next address.)
struct PagedLoader {
  const int32_t* row;  // the request's block-table row (uniform)
  int Hkv, kh, D, BS, NB, bs_shift;
  // physical block of the wave-uniform key nb
  __device__ __forceinline__ int block_of(int nb) const {
    return clampi(row[__builtin_amdgcn_readfirstlane(nb) >> bs_shift], 0, NB - 1);
  }
  // first element of kv head kh in the block holding key nb
  __device__ __forceinline__ size_t block_offset(int nb) const {
    return ((size_t)block_of(nb) * Hkv + kh) * BS * D;
  }
};

// scale_log2 > 0 always: the host folds a negative scale into negate_q (an exact sign flip of q)
// and replaces a zero scale by the smallest normal float (every score then rounds to 2^0 = 1).
template <int D, bool PAGED>
__global__ void __launch_bounds__(kPrefillThreads, 3)
prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
               const int32_t* __restrict__ qo_indptr, const int32_t* __restrict__ kv_indptr,
               const int32_t* __restrict__ kv_lens, const int32_t* __restrict__ tables,
               int Hq, int Hkv, int BS, int NB, int max_blocks, int causal, float scale_log2,
               int negate_q, int xcd_group, int xcd_heads, int n_rows, int bs_shift, int batch,
               int total_q, int total_kv, const uint32_t* __restrict__ order_dev,
               const TileOrder order, int hp) {
  using C = PrefillCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];
  // K ring at smem + j * TILE (j < 4), V ring after it; the output tile reuses the space

  // A work-group takes hp q heads of one kv head (hp = gcd(G, 4)) over 32 * 4 / hp query rows:
  // wave w serves head hs = w % hp, row block rb = w / hp.
  const int G = Hq / Hkv;
  const int bm = kPrefillWaves / hp * 32;  // query rows per work-group
  int hg, y;
  xcd_map(Hq / hp, Hkv, G / hp, xcd_group, xcd_heads, hg, y);
  if (y >= n_rows) return;
  TileWork tw;
  if (!resolve_tile<PAGED>(y, order, order_dev, qo_indptr, kv_indptr, kv_lens, batch, total_q,
                           total_kv, max_blocks * BS, bm, tw))
    return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = hg * hp + w % hp;
  const int rb = w / hp;
  const int b = tw.b;
  const int kh = (hg * hp) / G;
  const int q0 = tw.q0;
  const int qo = tw.qo;
  const int kv = tw.kv;
  const int64_t kv0 = tw.kv0;
  const int m0 = tw.qt * bm;
  const int off = kv - qo;  // row i sits at key position i + off

  // keys this tile can see: [0, kv_end)
  int kv_end = kv;
  if (causal) kv_end = min(kv, m0 + bm + off);
  const int n_kt = kv_end > 0 ? (kv_end + C::BN - 1) / C::BN : 0;

  const int qcol = lane & 31;   // query column of this lane
  const int half = lane >> 5;   // 0/1
  const int row = m0 + rb * 32 + qcol;     // query row within the request
  const bool row_ok = row < qo;

  // Q^T operand: lane holds Q[row][ks*16 + 8*half .. +8] (loaded after the first tiles, below)
  bf16x8 qreg[C::KS];

  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;  // log2 units
  float l_run = 0.f;
  // last visible key of this row: the causal limit and the ragged end in one bound
  const int lim = causal ? min(row + off, kv - 1) : kv - 1;

  const RaggedLoader rl{kv0, Hkv, kh, D};
  const PagedLoader pl{tables + (size_t)b * max_blocks, Hkv, kh, D, BS, NB, bs_shift};

  // Loads of one K or V tile (rows n0 .. n0+BN-1) straight into LDS: load instruction i of wave w
  // fills 1 KiB chunk j = i * waves + w of the tile, lane l its physical unit 64 j + l, i.e. row
  // rr = (64 j + l) / UPR, stored unit l % UPR, which holds logical unit (l % UPR) ^ swz(rr).
  // Rows past the request's end re-read its last row (their probabilities are exactly 0).
  const uint32_t lds0 = lds_addr(smem);
  const int pc = lane % C::UPR;
  // Per-lane byte offsets of a whole tile (no row past the request's end), the same for K and V
  // and for every such tile: computed once. (Paged: rows n0 + r sit at offset r & (BS-1) of their
  // block when BS divides the tile's first row, i.e. BS <= BN.)
  uint32_t vo_full[C::NL];
#pragma unroll
  for (int i = 0; i < C::NL; ++i) {
    const int rr = (i * kPrefillWaves + w) * C::ROWS_PER_LOAD + lane / C::UPR;
    const int cu = pc ^ swz<C::UPR>(rr);
    if constexpr (PAGED) vo_full[i] = (uint32_t)(__umul24(rr & (BS - 1), D) + cu * 8) * 2u;
    else vo_full[i] = (uint32_t)(__umul24(rr, Hkv * D) + cu * 8) * 2u;
  }
  const bool bs_in_tile = !PAGED || BS <= C::BN;
  auto load_tile = [&](const uint16_t* src, int t, uint32_t lds_tile) {
    const int n0 = t * C::BN;
    const int last_r = kv - 1 - n0;  // >= 0: the tile's last row inside the request
    if (bs_in_tile && n0 + C::BN <= kv) {
#pragma unroll
      for (int i = 0; i < C::NL; ++i) {
        const int j = i * kPrefillWaves + w;  // wave-uniform
        size_t base;
        if constexpr (PAGED) base = pl.block_offset(n0 + j * C::ROWS_PER_LOAD);
        else base = rl.row_offset(n0);
        dma_load16(src + base, vo_full[i], lds_tile + (uint32_t)j * 1024u);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < C::NL; ++i) {
      const int j = i * kPrefillWaves + w;                 // wave-uniform
      const int rr = j * C::ROWS_PER_LOAD + lane / C::UPR;
      const int cu = pc ^ swz<C::UPR>(rr);
      const int r = min(rr, last_r);
      size_t base;   // wave-uniform element offset
      uint32_t vo;   // per-lane byte offset
      if constexpr (PAGED) {
        // the instruction's first row: wave-uniform, in the same block as every row it loads
        const int nb = min(n0 + j * C::ROWS_PER_LOAD, kv - 1);
        base = pl.block_offset(nb);
        vo = (uint32_t)(__umul24((n0 + r) & (BS - 1), D) + cu * 8) * 2u;
      } else {
        base = rl.row_offset(n0);
        vo = (uint32_t)(__umul24(r, Hkv * D) + cu * 8) * 2u;  // 24-bit products (host-checked)
      }
      dma_load16(src + base, vo, lds_tile + (uint32_t)j * 1024u);
    }
  };
  auto k_lds_of = [&](int slot) { return lds0 + (uint32_t)(slot * C::TILE * 2); };
  auto v_lds_of = [&](int slot) { return lds0 + (uint32_t)((C::KBUF + slot) * C::TILE * 2); };

  // LDS read offsets (elements, within a tile). K as the A operand: row mt*32 + qcol, logical
  // unit 2 ks + half. V^T transpose reads: 16-lane group g reads key rows 4*(g/2) + (l%16)/4
  // (+8 for the second read) at columns 16*(g%2) + 4*(l%4) of each 32-wide d tile, i.e. logical
  // unit 4 dt + cq, element 4*(l%2) within it.
  const int swk = swz<C::UPR>(qcol);
  const int grp = lane >> 4;
  const int tr_row = 4 * (grp >> 1) + ((lane & 15) >> 2);
  const int cq = 2 * (grp & 1) + ((lane & 3) >> 1);
  const int sw_lo = swz<C::UPR>(tr_row), sw_hi = swz<C::UPR>(tr_row + 8);
  const int tr_lo = tr_row * D + 4 * (lane & 1);
  const int tr_hi = (tr_row + 8) * D + 4 * (lane & 1);

  // Pipeline, per wave: issue order K0 V0 K1 K2 | V1 K3 | V2 K4 | ... (step t issues V(t+1) and
  // K(t+3)); so before step t only K(t+2)'s NL loads may still be in flight (before step 0 also
  // K1's: waiting for them too is merely early).
  if (n_kt > 0) {
    load_tile(k, 0, k_lds_of(0));
    load_tile(v, 0, v_lds_of(0));
    if (n_kt > 1) load_tile(k, 1, k_lds_of(1));
    if (n_kt > 2) load_tile(k, 2, k_lds_of(2));
  }
  // q rows are loaded after the first tiles' loads are issued, so those queue first (2-3 % faster
  // on the ragged prefill than the other order)
  {
    const int r = row_ok ? row : (qo - 1);
    const uint16_t* qp = q + ((size_t)(q0 + r) * Hq + h) * D + 8 * half;
    const uint32_t flip = negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 x = load16(qp + ks * 16);
      x ^= u32x4{flip, flip, flip, flip};
      qreg[ks] = as_bf16x8(x);
    }
  }
  // last key any row of this wave can see (causal): tiles past it are skipped by the wave; a wave
  // whose rows all lie past the request's end (the q tile's padding) skips every tile
  const int wave_last_key = m0 + rb * 32 >= qo ? -1 : (causal ? m0 + rb * 32 + 31 + off : 0x7fffffff);
  for (int t = 0; t < n_kt; ++t) {
    const int n0 = t * C::BN;
    // tile t landed for every wave; every wave is done with tile t-1's buffers (K(t+3) reuses
    // K(t-1)'s slot, V(t+1) V(t-1)'s)
    if (t + 2 < n_kt) wait_vm_barrier<C::NL>();
    else wait_vm_barrier<0>();
    if (t + 1 < n_kt) load_tile(v, t + 1, v_lds_of((t + 1) & 1));
    if (t + 3 < n_kt) load_tile(k, t + 3, k_lds_of((t + 3) & 3));
    const uint16_t* const k_lds = smem + (t & 3) * C::TILE;
    const uint16_t* const v_lds = smem + (C::KBUF + (t & 1)) * C::TILE;
    if (n0 > wave_last_key) continue;

    // S^T tile: lane holds keys n0 + mt*32 + 8*(r/4) + 4*half + r%4 of query qcol (raw scores)
    f32x16 s[C::MT];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            k_lds + (mt * 32 + qcol) * D + (((2 * ks + half) ^ swk) << 3)));
        s[mt] = mfma32(a, qreg[ks], s[mt]);
      }
    sched_qk_pipeline<C::KS * C::MT, kQkAhead>();

    // mask only tiles crossing the ragged end or this wave's causal diagonal
    const bool need_mask = (n0 + C::BN > kv) || (causal && n0 + C::BN - 1 > m0 + rb * 32 + off);
    if (need_mask) {
      // key n0 + mt*32 + 8*(r/4) + 4*half + r%4 is visible iff mt*32 + 8*(r/4) + r%4 <= thr
      const int thr = lim - n0 - 4 * half;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mt * 32 + 8 * (r >> 2) + (r & 3) > thr) s[mt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
    mx = max_xor32(mx);
    const float tmax = mx * scale_log2;
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescaleLog2) != 0) {
      const float m_new = fmaxf(m_run, tmax);
      const float corr = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] *= corr;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
    float ps = 0.f;
    bf16x8 pb[C::PS];
#pragma unroll
    for (int st = 0; st < C::PS; ++st) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float e = fast_exp2(__builtin_fmaf(s[st >> 1][8 * (st & 1) + j], scale_log2, neg_m));
        pv[j] = e;
      }
      pb[st] = pack_bf16x8(pv);
      ps = sum_bf16x8(pb[st], ps);  // the sum of the probabilities PV actually uses
    }
    l_run += ps;

    // O^T += V^T P^T; k-index 8*half + j <-> key 16*st + 8*(j/4) + 4*half + j%4
#pragma unroll
    for (int st = 0; st < C::PS; ++st)
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const uint16_t* vt = v_lds + st * 16 * D;
        const u32x2 lo = lds_read_tr16(vt + tr_lo + (((4 * dt + cq) ^ sw_lo) << 3));
        const u32x2 hi = lds_read_tr16(vt + tr_hi + (((4 * dt + cq) ^ sw_hi) << 3));
        o[dt] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[st], o[dt]);
      }
  }

  // normalise, stage the wave's 32 rows in LDS, then write whole rows with 16-byte stores
  l_run = sum_xor32(l_run);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  __syncthreads();  // no tile loads in flight (the last step waited for all), no tile reads left
  uint16_t* const ost = smem + w * 32 * C::RSO;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = dt * 32 + 8 * g + 4 * half;
      *reinterpret_cast<u32x2*>(ost + qcol * C::RSO + d) =
          u32x2{pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
    }
  __syncthreads();
#pragma unroll
  for (int u = lane; u < 32 * C::UPR; u += kWave) {
    const int rr = u / C::UPR;
    const int cu = u - rr * C::UPR;
    const int orow = m0 + rb * 32 + rr;
    if (orow < qo)
      store16_nt(out + ((size_t)(q0 + orow) * Hq + h) * D + cu * 8,
              *reinterpret_cast<const u32x4*>(ost + rr * C::RSO + cu * 8));
  }
}
// ------------------------------------------------------------------------------------------------
// Variant with 16 query rows per wave on v_mfma_f32_16x16x32_bf16, for head_dim 256: a wave holds
// half the output accumulator and half the q rows of the 32-row form, so with one K / V tile of
// register prefetch it fits 168 VGPRs and three waves share a SIMD. The kernel is bound by
// latency (LDS reads feeding each MFMA, the per-tile barrier), not by a unit's throughput, so the
// third wave per SIMD is what hides it: 12 waves x 16 rows measured 10 % faster than 8 waves with
// two tiles of prefetch. Each wave still reads the whole K / V tile from LDS, so LDS traffic per
// FLOP is twice the 32-row form's.
//   S^T = K Q^T per 16-key tile: A = 16 K rows x 32 d (LDS), B = the wave's Q rows (registers);
//     lane l holds keys 16*kt + 4*(l/16) + r of query l%16.
//   O^T += V^T P^T per 32-key step: the lane's 8 probabilities (keys 4*(l/16) + j and
//     16 + 4*(l/16) + j of the step) are its B operand as they stand; the A operand takes V^T
//     with the same key order from two LDS transpose reads.
// 12 waves x 16 rows serve hp q heads of one kv head (hp = gcd(G, 12)) over a q tile of 192 / hp
// rows: with 16 q / 4 kv heads, four heads over 48 rows. The heads share every K / V tile the work-
// group stages, the waves' causal extents differ by at most a tile height, and a request's last,
// partial q tile keeps fewer waves idle than a 192-row tile of one head did (455 -> 421 us on the
// chunked prefill workload, same box). The first 8 waves load and stage the K / V tiles (a 32-key
// tile is 1024 16-byte units: two per loading thread).
constexpr int kP16Waves = 12;
constexpr int kP16Threads = kP16Waves * kWave;
constexpr int kP16LoadThreads = 8 * kWave;  // threads that load and stage K / V tiles
constexpr int kP16BM = 16 * kP16Waves;  // query rows per work-group

template <int D>
struct P16Cfg {
  static constexpr int BN = (D >= 256) ? 32 : 64;  // keys per kv tile
  static constexpr int KT = BN / 16;               // 16-key tiles of S^T
  static constexpr int KS = D / 32;                // 32-wide d steps of QK^T
  static constexpr int PS = BN / 32;               // 32-key steps of PV
  static constexpr int DT = D / 16;                // 16-wide d tiles of O^T
  // LDS row strides in elements, chosen by measurement (a sweep of K pads 16..80 bytes by V pads
  // 32..224 bytes): a 32-byte pad on K rows leaves the K operand reads free of bank conflicts
  // (SQ_LDS_BANK_CONFLICT ~0; a 16-byte pad conflicts), and with a 96-byte pad on V rows the
  // kernel ran 7 % faster than with the 16 / 32-byte pads it had before.
  static constexpr int RSE = D + 16;               // K rows and the output tile
  static constexpr int RSV = D + 48;               // V rows
  static constexpr int BUF = BN * (RSE + RSV);     // one K+V tile buffer
  static constexpr int UPR = D / 8;                // 16-byte units per row
  static constexpr int UNITS = BN * UPR;           // units per tile (K or V)
  static constexpr int UPT = UNITS / kP16LoadThreads;  // units per loading thread
  static constexpr int PF = 1;                     // kv tiles in flight in registers
  static constexpr int LDS_ELEMS = (2 * BUF > kP16BM * RSE) ? 2 * BUF : kP16BM * RSE;
  static_assert(UNITS % kP16LoadThreads == 0, "tile units must divide evenly");
  static_assert(kWave / UPR <= 16, "a wave's load rows must stay inside one block");
};

template <int D, bool PAGED>
__global__ void __launch_bounds__(kP16Threads, kP16Waves / 4)
prefill16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
                 const int32_t* __restrict__ qo_indptr, const int32_t* __restrict__ kv_indptr,
                 const int32_t* __restrict__ kv_lens, const int32_t* __restrict__ tables,
                 int Hq, int Hkv, int BS, int NB, int max_blocks, int causal, float scale_log2,
                 int negate_q, int xcd_group, int xcd_heads, int n_rows, int bs_shift, int batch,
                 int total_q, int total_kv, const uint32_t* __restrict__ order_dev,
                 const TileOrder order, int hp) {
  using C = P16Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];
  // buffer j (0/1): K rows at smem + j*BUF, V rows BN*RSE further; the output tile reuses it

  // A work-group takes hp q heads of one kv head (hp = gcd(G, 12)) over 16 * 12 / hp query rows:
  // wave w serves head hs = w % hp, row block rb = w / hp.
  const int G = Hq / Hkv;
  const int bm = kP16Waves / hp * 16;  // query rows per work-group
  int hg, y;
  xcd_map(Hq / hp, Hkv, G / hp, xcd_group, xcd_heads, hg, y);
  if (y >= n_rows) return;
  TileWork tw;
  if (!resolve_tile<PAGED>(y, order, order_dev, qo_indptr, kv_indptr, kv_lens, batch, total_q,
                           total_kv, max_blocks * BS, bm, tw))
    return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = hg * hp + w % hp;
  const int rb = w / hp;
  const int b = tw.b;
  const int kh = (hg * hp) / G;
  const int q0 = tw.q0;
  const int qo = tw.qo;
  const int kv = tw.kv;
  const int64_t kv0 = tw.kv0;
  const int m0 = tw.qt * bm;
  const int off = kv - qo;  // row i sits at key position i + off

  int kv_end = kv;
  if (causal) kv_end = min(kv, m0 + bm + off);
  const int n_kt = kv_end > 0 ? (kv_end + C::BN - 1) / C::BN : 0;

  const int qcol = lane & 15;  // query of this lane within the wave
  const int grp = lane >> 4;   // 0..3
  const int row = m0 + rb * 16 + qcol;
  const bool row_ok = row < qo;

  // Q^T operand: lane holds Q[row][32*ks + 8*grp .. +8]
  bf16x8 qreg[C::KS];
  {
    const int r = row_ok ? row : (qo - 1);
    const uint16_t* qp = q + ((size_t)(q0 + r) * Hq + h) * D + 8 * grp;
    const uint32_t flip = negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 x = load16(qp + ks * 32);
      x ^= u32x4{flip, flip, flip, flip};
      qreg[ks] = as_bf16x8(x);
    }
  }

  f32x4 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // log2 units
  float l_run = 0.f;
  const int lim = causal ? min(row + off, kv - 1) : kv - 1;

  const RaggedLoader rl{kv0, Hkv, kh, D};
  const PagedLoader pl{tables + (size_t)b * max_blocks, Hkv, kh, D, BS, NB, bs_shift};

  u32x4 kpre[C::PF][C::UPT], vpre[C::PF][C::UPT];
  const int w_u0 = __builtin_amdgcn_readfirstlane(tid & ~63);  // first unit of this wave
  // Loads of tile rows n0 .. n0+BN-1; rows past the request's end re-read its last row (their
  // probabilities are exactly 0). Every call issues the same loads in the same order, whatever
  // n0 is, so the wait before each stage counts exactly the loads still needed.
  const int last_n0 = (n_kt - 1) * C::BN;  // first row of the last tile
  const bool loader = w < kP16LoadThreads / kWave;  // wave-uniform
  // Paged: the physical blocks a fetch reads are looked up one fetch ahead, so the block-table
  // reads (scalar loads) complete under the wait that precedes the next barrier instead of
  // stalling the fetch that needs them.
  int blk_next[C::UPT];
  auto lookup = [&](int n0) {
    if constexpr (PAGED) {
      n0 = __builtin_amdgcn_readfirstlane(min(n0, last_n0));
#pragma unroll
      for (int i = 0; i < C::UPT; ++i)  // raw entries: clamped where they are used
        blk_next[i] = pl.row[(min(n0 + (i * kP16LoadThreads + w_u0) / C::UPR, kv - 1)) >> bs_shift];
    }
  };
  auto fetch = [&](int n0, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
    if (!loader) return;
    n0 = __builtin_amdgcn_readfirstlane(min(n0, last_n0));  // past the last tile: repeat it
    const int last_r = kv - 1 - n0;  // >= 0: the tile's last row inside the request
#pragma unroll
    for (int i = 0; i < C::UPT; ++i) {
      const int u = i * kP16LoadThreads + tid;
      const int rr = u / C::UPR;
      const int cu = u - rr * C::UPR;
      const int r = min(rr, last_r);
      size_t base;  // wave-uniform element offset
      int off;      // per-lane byte offset
      if constexpr (PAGED) {
        // the instruction's first row is wave-uniform and in the same block as every row it
        // loads; its block was looked up by the previous fetch
        base = ((size_t)clampi(blk_next[i], 0, NB - 1) * Hkv + kh) * BS * D;
        off = (__umul24((n0 + r) & (BS - 1), D) + cu * 8) * 2;  // 24-bit products (host-checked)
      } else {
        base = rl.row_offset(n0);
        off = (__umul24(r, Hkv * D) + cu * 8) * 2;
      }
      kpre[sl][i] = buffer_load16(buffer_at(k + base), off);
      vpre[sl][i] = buffer_load16(buffer_at(v + base), off);
      memory_order_point();
    }
    lookup(n0 + C::BN);
  };
  auto stash = [&](int buf, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
    if (!loader) return;
    uint16_t* const k_lds = smem + buf * C::BUF;
    uint16_t* const v_lds = k_lds + C::BN * C::RSE;
#pragma unroll
    for (int i = 0; i < C::UPT; ++i) {
      const int u = i * kP16LoadThreads + tid;
      const int rr = u / C::UPR;
      const int cu = u - rr * C::UPR;
      *reinterpret_cast<u32x4*>(k_lds + rr * C::RSE + cu * 8) = kpre[sl][i];
      *reinterpret_cast<u32x4*>(v_lds + rr * C::RSV + cu * 8) = vpre[sl][i];
    }
  };

  // V^T transpose reads: lane i of 16-lane group grp addresses key row 4*grp + i/4 (+16 for the
  // second read) at d columns 4*(i%4) .. +3 of each 16-wide d tile.
  const int tr_off = (4 * grp + ((lane & 15) >> 2)) * C::RSV + 4 * (lane & 3);

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, (C::PF > 1) ? 1 : 0>;
  if (n_kt > 0) {
    if (loader) lookup(0);
    fetch(0, S0{});
    stash(0, S0{});
    fetch(C::BN, S1{});
    if constexpr (C::PF > 1) fetch(2 * C::BN, S0{});
  }
  const int wave_first_row = m0 + rb * 16;
  // tiles past the last key a row of this wave sees are skipped, all of them by a wave whose rows
  // lie past the request's end (the q tile's padding)
  const int wave_last_key =
      wave_first_row >= qo ? -1 : (causal ? wave_first_row + 15 + off : 0x7fffffff);
  auto step = [&](int t, auto slot_c) {
    const int n0 = t * C::BN;
    __syncthreads();  // tile t staged by every wave; tile t-1's buffer no longer read
    const uint16_t* const k_lds = smem + (t & 1) * C::BUF;
    const uint16_t* const v_lds = k_lds + C::BN * C::RSE;
    if (n0 <= wave_last_key) {
      f32x4 s[C::KT];
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
              k_lds + (kt * 16 + qcol) * C::RSE + ks * 32 + 8 * grp));
          s[kt] = mfma16(a, qreg[ks], s[kt]);
        }
      sched_qk_pipeline<C::KS * C::KT, kQkAhead>();
      const bool need_mask =
          (n0 + C::BN > kv) || (causal && n0 + C::BN - 1 > wave_first_row + off);
      if (need_mask) {
        // key n0 + 16*kt + 4*grp + r is visible iff 16*kt + r <= thr
        const int thr = lim - n0 - 4 * grp;
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kt + r > thr) s[kt][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kt][r]);
      mx = max_xor32(max_xor16(mx));
      const float tmax = mx * scale_log2;
      if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescaleLog2) != 0) {
        const float m_new = fmaxf(m_run, tmax);
        const float corr = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= corr;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) o[dt] *= corr;
      }
      const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
      float ps = 0.f;
      bf16x8 pb[C::PS];
#pragma unroll
      for (int st = 0; st < C::PS; ++st) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e =
              fast_exp2(__builtin_fmaf(s[2 * st + (j >> 2)][j & 3], scale_log2, neg_m));
          pv[j] = e;
        }
        pb[st] = pack_bf16x8(pv);
        ps = sum_bf16x8(pb[st], ps);
      }
      l_run += ps;
#pragma unroll
      for (int st = 0; st < C::PS; ++st)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const uint16_t* vp = v_lds + st * 32 * C::RSV + dt * 16 + tr_off;
          const u32x2 lo = lds_read_tr16(vp);
          const u32x2 hi = lds_read_tr16(vp + 16 * C::RSV);
          o[dt] = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[st], o[dt]);
        }
    }
    // Unconditional, also after the last tile (a stage nobody reads, loads of clamped rows), so
    // every path into the next step has issued the same loads.
    stash((t + 1) & 1, slot_c);
    fetch(n0 + (1 + C::PF) * C::BN, slot_c);
  };
  if (n_kt > 0) {
    if constexpr (C::PF == 1) {
      int t = 0;
      do {
        step(t, S0{});
      } while (++t < n_kt);
    } else {
      for (int t = 0;; t += 2) {
        step(t, S1{});
        if (t + 1 >= n_kt) break;
        step(t + 1, S0{});
        if (t + 2 >= n_kt) break;
      }
    }
  }

  // normalise, stage the wave's 16 rows in LDS, then write whole rows with 16-byte stores
  l_run = sum_xor32(sum_xor16(l_run));
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  __syncthreads();
  uint16_t* const ost = smem + w * 16 * C::RSE;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int d = dt * 16 + 4 * grp;
    *reinterpret_cast<u32x2*>(ost + qcol * C::RSE + d) =
        u32x2{pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
              pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
  }
  __syncthreads();
#pragma unroll
  for (int u = lane; u < 16 * C::UPR; u += kWave) {
    const int rr = u / C::UPR;
    const int cu = u - rr * C::UPR;
    const int orow = wave_first_row + rr;
    if (orow < qo)
      store16_nt(out + ((size_t)(q0 + orow) * Hq + h) * D + cu * 8,
              *reinterpret_cast<const u32x4*>(ost + rr * C::RSE + cu * 8));
  }
}

// head dims that run the 16-row form (at head_dim <= 128 the 32-row form is faster: two waves per
// SIMD fit either way, and it reads half the LDS bytes per FLOP)
template <int D>
constexpr bool use_p16() {
  return D >= 256;
}

// Keys a (request, q tile)'s rows can see: the work the longest-first schedule sorts by.
static int64_t tile_work(int qo, int64_t kv, int qt, int causal, int bm) {
  int64_t vis = kv;
  if (causal) vis = std::min<int64_t>(kv, (int64_t)(qt + 1) * bm + kv - qo);
  return std::max<int64_t>(vis, 0);
}

// q heads per work-group of the head_dim-256 form: the largest count that divides both the group
// size and its 12 waves
int prefill16_heads(int group) {
  int a = group, b = kP16Waves;
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// q heads per work-group of the head_dim <= 128 form: the largest count dividing the group size
// and its 4 waves
int prefill_heads(int group) { return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1); }

int prefill_tile_rows(int head_dim, int group) {
  return head_dim >= 256 ? kP16BM / prefill16_heads(group) : kBM / prefill_heads(group);
}

int64_t prefill_tile_count(int batch, const int32_t* qo_indptr_h, int bm) {
  int64_t n = 0;
  for (int b = 0; b < batch; ++b) n += (qo_indptr_h[b + 1] - qo_indptr_h[b] + bm - 1) / bm;
  return n;
}

static size_t align256p(size_t x) { return (x + 255) & ~(size_t)255; }

size_t prefill_workspace_bytes(int64_t tiles) {
  return tiles <= kMaxOrder ? 0 : align256p((size_t)tiles * sizeof(uint32_t));
}

// Schedule of the (request, q tile) work-groups from the host copies of the lengths, for launches
// of at most kMaxOrder tiles (passed by value with the launch).
//
// lists == 1: all tiles longest-first. lists > 1: rows y and y' run their head groups on the same
// XCDs iff y == y' (mod lists) (the XCD mapping of the launch), so each request is kept on one
// row class: requests are dealt to the classes longest-processing-time first (by their total
// work), and a class holds its requests in order of their longest tile, each request's tiles
// together and shortest-first. The tiles of one request then run side by side on one XCD and walk
// the same K/V prefix through its L2 instead of fetching it again from HBM. (Shortest-first within
// a request: the chunked prefill workload read 290 MB per call against 321 MB longest-first, in
// the same time; ordering the requests by total work or by tile count ran 5-13 % slower.) Classes
// are interleaved row by row and padded with kNoTile to equal length; if that padding would
// overflow the by-value list, the plain longest-first order is used.
static void build_order(const PrefillArgs& a, int lists, TileOrder& ord) {
  struct Item {
    int64_t work;
    uint32_t e;
  };
  struct Req {
    int64_t total = 0, longest = 0;
    int b = 0;
    std::vector<Item> tiles;
  };
  std::vector<Req> reqs;
  std::vector<Item> items;
  for (int b = 0; b < a.batch; ++b) {
    const int qo = a.qo_indptr_h[b + 1] - a.qo_indptr_h[b];
    const int64_t kv = a.kv_indptr_h ? (int64_t)a.kv_indptr_h[b + 1] - a.kv_indptr_h[b]
                                     : std::min<int64_t>(std::max(a.kv_lens_h[b], 0),
                                                         (int64_t)a.max_blocks_per_seq * a.block_size);
    const int n_qt = (qo + a.tile_rows - 1) / a.tile_rows;
    if (n_qt == 0) continue;
    Req r;
    r.b = b;
    for (int qt = 0; qt < n_qt; ++qt) {
      const Item it{tile_work(qo, kv, qt, a.causal, a.tile_rows), ((uint32_t)b << 16) | (uint32_t)qt};
      r.tiles.push_back(it);
      items.push_back(it);
      r.total += it.work;
      r.longest = std::max(r.longest, it.work);
    }
    reqs.push_back(std::move(r));
  }
  auto longest_first = [](const Item& x, const Item& y) { return x.work > y.work; };
  auto plain = [&]() {
    std::stable_sort(items.begin(), items.end(), longest_first);
    for (size_t i = 0; i < items.size(); ++i) ord.e[i] = items[i].e;
    ord.n = (int)items.size();
  };
  if (lists <= 1 || (int)reqs.size() < 2) return plain();
  // deal requests to classes, largest total first, each to the least loaded class
  std::vector<size_t> by_total(reqs.size());
  for (size_t i = 0; i < reqs.size(); ++i) by_total[i] = i;
  std::stable_sort(by_total.begin(), by_total.end(),
                   [&](size_t x, size_t y) { return reqs[x].total > reqs[y].total; });
  std::vector<int64_t> load(lists, 0);
  std::vector<std::vector<size_t>> cls(lists);
  for (size_t i : by_total) {
    const int c = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[c] += reqs[i].total;
    cls[c].push_back(i);
  }
  size_t len = 0;
  for (auto& c : cls) {
    std::stable_sort(c.begin(), c.end(),
                     [&](size_t x, size_t y) { return reqs[x].longest > reqs[y].longest; });
    size_t n = 0;
    for (size_t i : c) n += reqs[i].tiles.size();
    len = std::max(len, n);
  }
  if (len * lists > (size_t)kMaxOrder) return plain();
  for (int c = 0; c < lists; ++c) {
    size_t j = 0;
    for (size_t i : cls[c]) {
      std::vector<Item>& t = reqs[i].tiles;
      std::stable_sort(t.begin(), t.end(),
                       [](const Item& x, const Item& y) { return x.work < y.work; });
      for (const Item& it : t) ord.e[(j++) * lists + c] = it.e;
    }
    for (; j < len; ++j) ord.e[j * lists + c] = kNoTile;
  }
  ord.n = (int)(len * lists);
}

// Device-built longest-first schedule for launches of more tiles than the by-value list holds:
// one work-group counts the tiles per work bucket (visible keys in units of 32, most first),
// scans the counts and scatters each tile's entry to its bucket's range of the workspace. Tiles
// of one bucket land in any order (each tile's result does not depend on its slot). Entries
// [device tile count, capacity) read kNoTile; tiles beyond capacity (device offsets that
// disagree with their host copies) are dropped.
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 4096;
constexpr int kPlanPerThread = kPlanBuckets / kPlanThreads;

__global__ void __launch_bounds__(kPlanThreads)
prefill_plan_kernel(const int32_t* __restrict__ qo_indptr, const int32_t* __restrict__ kv_indptr,
                    const int32_t* __restrict__ kv_lens, int batch, int causal, int total_q,
                    int total_kv, int kv_cap, int bm, uint32_t* __restrict__ order, int capacity) {
  __shared__ int hist[kPlanBuckets];
  __shared__ int wave_sum[kPlanThreads / kWave];
  const int tid = threadIdx.x;
  for (int i = tid; i < kPlanBuckets; i += kPlanThreads) hist[i] = 0;
  __syncthreads();
  auto extents = [&](int b, int& qo, int& kv) {
    const int q0 = clampi(qo_indptr[b], 0, total_q);
    qo = clampi(qo_indptr[b + 1], q0, total_q) - q0;
    if (kv_lens != nullptr) {
      kv = clampi(kv_lens[b], 0, kv_cap);
    } else {
      const int k0 = clampi(kv_indptr[b], 0, total_kv);
      kv = clampi(kv_indptr[b + 1], k0, total_kv) - k0;
    }
  };
  auto bucket = [&](int qo, int kv, int qt) {
    int vis = kv;
    if (causal) vis = (int)clampi<int64_t>((int64_t)(qt + 1) * bm + kv - qo, 0, kv);
    return kPlanBuckets - 1 - min((vis + 31) >> 5, kPlanBuckets - 1);
  };
  for (int b = tid; b < batch; b += kPlanThreads) {
    int qo, kv;
    extents(b, qo, kv);
    const int n_qt = min((qo + bm - 1) / bm, 0xffff);
    for (int qt = 0; qt < n_qt; ++qt) atomicAdd(&hist[bucket(qo, kv, qt)], 1);
  }
  __syncthreads();
  // exclusive scan: each thread owns kPlanPerThread consecutive buckets
  int local[kPlanPerThread];
  int run = 0;
#pragma unroll
  for (int j = 0; j < kPlanPerThread; ++j) {
    local[j] = run;
    run += hist[tid * kPlanPerThread + j];
  }
  const int lane = tid & (kWave - 1);
  int incl = run;
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    const int o = __shfl_up(incl, s, kWave);
    if (lane >= s) incl += o;
  }
  if (lane == kWave - 1) wave_sum[tid / kWave] = incl;
  __syncthreads();
  int before = 0;
  for (int wv = 0; wv < tid / kWave; ++wv) before += wave_sum[wv];
  int total = 0;
  for (int wv = 0; wv < kPlanThreads / kWave; ++wv) total += wave_sum[wv];
  const int start = before + incl - run;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPlanPerThread; ++j) hist[tid * kPlanPerThread + j] = start + local[j];
  __syncthreads();
  for (int b = tid; b < batch; b += kPlanThreads) {
    int qo, kv;
    extents(b, qo, kv);
    const int n_qt = min((qo + bm - 1) / bm, 0xffff);
    for (int qt = 0; qt < n_qt; ++qt) {
      const int pos = atomicAdd(&hist[bucket(qo, kv, qt)], 1);
      if (pos < capacity) order[pos] = ((uint32_t)b << 16) | (uint32_t)qt;
    }
  }
  for (int i = total + tid; i < capacity; i += kPlanThreads) order[i] = kNoTile;
}

template <int D, bool PAGED>
static hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t stream) {
  if (a.tiles == 0) return hipSuccess;
  // hp q heads of one kv head per work-group; the XCD mapping runs over the Hq / hp head groups
  const int hp = use_p16<D>() ? prefill16_heads(a.num_q_heads / a.num_kv_heads)
                              : prefill_heads(a.num_q_heads / a.num_kv_heads);
  const int hgs = a.num_q_heads / hp;
  const bool g8 = hgs % 8 == 0;
  const int xcd_group = (g8 && 8 % a.num_kv_heads == 0) ? 8 / a.num_kv_heads : 0;
  const int xcd_heads = (g8 && xcd_group == 0) ? hgs / 8 : 0;
  // rows whose head groups share XCDs: y mod row_classes (grouped mapping: the rows of a group;
  // plain mapping with hgs dividing 8: linear id y * hgs + x puts row y on XCDs (y % (8 / hgs)) *
  // hgs + x)
  const int row_classes = xcd_group > 0 ? xcd_group : ((!g8 && 8 % hgs == 0) ? 8 / hgs : 1);
  TileOrder order;
  order.n = 0;
  const uint32_t* order_dev = nullptr;
  const int kv_cap = PAGED ? a.max_blocks_per_seq * a.block_size : 0;
  int n_rows = (int)a.tiles;
  if (a.tiles <= kMaxOrder) {
    build_order(a, row_classes, order);
    n_rows = order.n;
  } else {
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.qo_indptr,
                       a.kv_indptr, a.kv_lens, a.batch, a.causal, a.total_q, (int)a.total_kv, kv_cap,
                       a.tile_rows, (uint32_t*)a.workspace, (int)a.tiles);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    order_dev = (const uint32_t*)a.workspace;
  }
  const int grid_rows = xcd_group > 0 ? (n_rows + xcd_group - 1) / xcd_group * xcd_group : n_rows;
  float scale_log2 = a.scale * kLog2e;
  const int negate_q = scale_log2 < 0.f;
  if (negate_q) scale_log2 = -scale_log2;
  if (!(scale_log2 >= 1.17549435e-38f)) scale_log2 = 1.17549435e-38f;  // zero (or denormal) scale
  const dim3 grid(hgs, grid_rows, 1);
  const int bs_shift = a.block_size > 0 ? __builtin_ctz((unsigned)a.block_size) : 0;
  if constexpr (use_p16<D>()) {
    hipLaunchKernelGGL((prefill16_kernel<D, PAGED>), grid, dim3(kP16Threads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.out, a.qo_indptr, a.kv_indptr, a.kv_lens, a.block_tables,
                       a.num_q_heads, a.num_kv_heads, a.block_size, a.num_blocks,
                       a.max_blocks_per_seq, a.causal, scale_log2, negate_q, xcd_group, xcd_heads,
                       n_rows, bs_shift, a.batch, a.total_q, (int)a.total_kv, order_dev, order, hp);
  } else {
    hipLaunchKernelGGL((prefill_kernel<D, PAGED>), grid, dim3(kPrefillThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.out, a.qo_indptr, a.kv_indptr, a.kv_lens, a.block_tables,
                       a.num_q_heads, a.num_kv_heads, a.block_size, a.num_blocks,
                       a.max_blocks_per_seq, a.causal, scale_log2, negate_q, xcd_group, xcd_heads,
                       n_rows, bs_shift, a.batch, a.total_q, (int)a.total_kv, order_dev, order, hp);
  }
  return hipGetLastError();
}

template <bool PAGED>
static hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_prefill_d<64, PAGED>(a, stream);
    case 128: return launch_prefill_d<128, PAGED>(a, stream);
    case 256: return launch_prefill_d<256, PAGED>(a, stream);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_ragged_prefill(const PrefillArgs& a, hipStream_t stream) {
  return launch_prefill<false>(a, stream);
}

hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t stream) {
  return launch_prefill<true>(a, stream);
}

}  // namespace pkv
