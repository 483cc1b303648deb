// Tiled exact attention forward, bf16 in / bf16 out, fp32 accumulation, for gfx950 (MI355X).
//
// Method: Q/K/V tiling with a running row maximum m, a running denominator l and a rescaled partial
// output O ("FlashAttention Explained: How AI Models Process Attention Faster and Use Less Memory",
// "How FlashAttention Works", parts 1-3; "Flash Attention Explained: Same Maths, Far Less Memory",
// "The idea: never materialise the matrix").  For each tile of keys and each query row i:
//   x_ij = s_ij * c  (c = |scale| * log2 e: exp2 with log2 e folded into the scale is the same exp)
//   m' = max(m, max_j x_ij),  p_ij = 2^(x_ij - m'),  l = 2^(m - m') l + sum_j p_ij,
//   O = 2^(m - m') O + sum_j p_ij v_j;   at the end O / l and LSE = ln2 * (m + log2 l).
// The reference maximum m is set from the first tile and afterwards moved only when a tile's weights
// 2^(x - m) would exceed 2^64; other tiles skip the max reduction entirely and O, l are rescaled only
// on those rare moves.  O / l and the LSE do not depend on which reference is used (exact arithmetic),
// and 2^64 keeps every sum far from fp32 overflow.  O is normalised by the sum of the same bf16
// weights that entered the value product (so a dominant weight cancels exactly), the LSE by the fp32
// sum.  The score tile lives only in registers.
//
// gfx950 mapping: 32 query rows per wave, two waves per SIMD (one wave's softmax runs while the other's
// MFMAs run; s_setprio favours the wave that is in an MFMA phase): 4 waves per (batch*head, 128-query
// tile) and two work-groups per CU, or, for large d = 128 grids without splits, 8 waves per 256-query
// tile and one work-group per CU.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS = A operand, Q^T in VGPRs = B operand): in
//    the 32x32 result a lane holds one query and 16 keys; lanes l and l^32 together hold the row, so
//    row max / row sum are in-lane reductions plus one v_permlane32_swap.
//  * O^T = V^T P^T on the same instruction: P^T (B operand) is the lane's own score registers
//    rounded to bf16, keys contracted in the order the score layout gives them; V^T (A operand) is
//    read from row-major V in LDS with ds_read_b64_tr_b16, whose 16-lane transpose delivers 4 keys at
//    one d per lane, in exactly that key order.
//  * K and V tiles of 64 keys go global -> LDS with direct 16-byte loads (buffer_load_dwordx4 ... lds,
//    no staging registers), double-buffered with one barrier per tile: tile t+1 is in flight while
//    tile t is computed.  The loads of tile t+1 are issued right after the S MFMAs of tile t (and the
//    V^T fragment reads), so they land during the softmax rather than during fragment reads; decode-like
//    launches (NT, below) issue them at the top of the tile.  16-byte chunks are XOR-swizzled within
//    each row (the swizzle is applied through each lane's source address) so every fragment read hits
//    distinct banks, and fragment addresses are per-lane bases plus compile-time offsets.
//  * Fragment reads run ahead of their MFMAs: K fragments four deep (scheduling groups), and all V^T
//    fragments of a tile are read before its softmax, so their LDS latency passes under the vector work.
//  * Causal tiles above the diagonal are never loaded; a wave skips the math of tiles that lie fully
//    above its rows; only diagonal and ragged-tail tiles evaluate the mask.
//  * Work-group ids are remapped so each XCD walks contiguous (head, tile) ranges, heaviest causal
//    query tiles first.  Causal grids of at least two work-groups per CU pair query tiles n-1-j and j in
//    one work-group (two passes over the same code), so every work-group carries the same load.
// Modes (template flags): SPLIT cuts each query tile's keys into S ranges of whole tiles, one
// work-group each, and writes fp32 partials (O_s normalised, LSE_s) that the decode combine merges; it
// serves short query chunks against a long cache and grouped-head decode (the G query heads of a
// key/value head are its query rows).  PAGED (with SPLIT, no mask) reads K and V through a block table
// from a page pool.  NT gives the K / V loads the non-temporal policy when one query tile reads them.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lds_tiles.h"

namespace fa {

struct PrefillParams {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  uint16_t* __restrict__ o;
  float* __restrict__ lse;
  int Nq, Nkv, off, n_qt, total;
  float c;        // max(|scale| * log2(e), 2^-126): strictly positive so masked -inf scores give 2^-inf = 0
  uint32_t qxor;  // 0x80008000 when scale < 0: q is negated on load (exact) so that c > 0
  // split-KV mode: key tiles [s*split_tiles, (s+1)*split_tiles) per work-group, partials into the workspace
  int S, split_tiles;
  float* __restrict__ ws_o;    // [B*H*N_q, S, D] fp32, O_s normalised
  float* __restrict__ ws_lse;  // [B*H*N_q, S] fp32, natural log; -inf for a row with no key in the range
  // paged key/value cache (split mode, no mask): k, v are page pools [num_pages, H, 2^lg_page, D] (H here
  // counts key/value heads), token t of sequence b is row t % 2^lg_page of page table[b][t >> lg_page], and
  // the sequence has min(max(seq_lens[b], 0), max_blocks << lg_page) tokens.
  const int* __restrict__ table;
  const int* __restrict__ seq_lens;
  int Hkv, num_pages, max_blocks, lg_page;
  int pair;  // causal, unsplit: work-group j runs query tile n_qt-1-j, then tile j (set by the launcher)
};

#ifndef FA_BC
#define FA_BC 64
#endif
constexpr float kBig = 0x1p64f;  // weights above this trigger a move of the reference maximum
// instruction classes of __builtin_amdgcn_sched_group_barrier, and the K fragment read-ahead
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
constexpr int kKDepth = 4;

template <int D, int NWAVES = 4>
struct Cfg {
  static constexpr int NW = NWAVES;        // waves per work-group
  static constexpr int NT = NW * 64;       // threads
  static constexpr int BR = NW * 32;       // query rows per work-group (32 per wave)
  static constexpr int BC = FA_BC;         // keys per tile
  static constexpr int NBLK = BC / 32;     // 32-key score blocks per tile
  static constexpr int ROWB = 2 * D;       // bytes per K / V row
  static constexpr int CH = D / 8;         // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;  // bytes per K (or V) tile
  static constexpr int STAGEB = 2 * TILEB; // K tile then V tile
  static constexpr int NSTAGE = 2;
  static constexpr int LPT = TILEB / (NT * 16);  // 16-byte direct loads per thread per tile (each of K, V)
  static constexpr int RPL = 1024 / ROWB;  // rows covered by one wave-wide 1 KB load
  static constexpr int KS = D / 16;        // MFMA k-steps over d
  static constexpr int MBD = D / 32;       // 32-wide d blocks of O^T
  static_assert(TILEB % (NT * 16) == 0, "tile loads must divide evenly");
  // fragment reads use 16-bit immediate offsets when NSTAGE * STAGEB <= 64 KB
};

// acc + sum of the 8 bf16 values of a fragment (v_dot2_f32_bf16 against ones).
__device__ __forceinline__ float sum_bf16x8(bf16x8 p, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pp = {p[2 * i], p[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pp, one, acc, false);
  }
  return acc;
}

// NT: K and V are read by exactly one work-group (one query tile per head, as in decode), so their loads
// use the non-temporal policy (measured +8% on grouped-head decode) instead of staying in the caches for
// the other query tiles of the head.
// NW: waves per work-group, 4 (two work-groups per CU) or 8 (one per CU; used where it measured faster)
template <int D, bool CAUSAL, bool SPLIT, bool PAGED = false, bool NT = false, int NW = 4>
__global__ __launch_bounds__(NW * 64, (NW == 8 ? 1 : 2)) void prefill_bf16_kernel(PrefillParams p) {
  static_assert(!PAGED || (SPLIT && !CAUSAL), "the paged cache is read by the unmasked split mode only");
  auto load16_lds = [](__amdgpu_buffer_rsrc_t r, int voff, void* lds_block) {
    if constexpr (NT)
      load_lds16_nt(r, voff, lds_block);
    else
      load_lds16(r, voff, lds_block);
  };
  using C = Cfg<D, NW>;
  // One LDS array per stage and operand: the compiler can then tell that the direct loads into one
  // stage do not alias the fragment reads of the other, and does not wait for those loads before them.
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[C::TILEB], lds_v0[C::TILEB], lds_k1[C::TILEB], lds_v1[C::TILEB];
  auto kbuf = [&](int st) -> uint8_t* { return st == 0 ? lds_k0 : lds_k1; };
  auto vbuf = [&](int st) -> uint8_t* { return st == 0 ? lds_v0 : lds_v1; };

  const int lid = xcd_logical_id(blockIdx.x, p.total);
  // Paired causal tiles: query tile i sees about i + 1 key blocks, so tiles n_qt-1-j and j together cost
  // the same for every j.  Without pairing the longest tiles set the end of a grid that spans a few
  // rounds of resident work-groups; with it every work-group carries the same load.
  const bool pair = CAUSAL && !SPLIT && p.pair;
  const int per_bh = SPLIT ? p.n_qt * p.S : (pair ? (p.n_qt + 1) / 2 : p.n_qt);
  const int bh = lid / per_bh;
  int qt_lo = lid - bh * per_bh, split = 0;
  if (SPLIT) {
    split = qt_lo % p.S;
    qt_lo /= p.S;
  }
  const int qt_hi = CAUSAL ? p.n_qt - 1 - qt_lo : qt_lo;  // heaviest query tiles first
  const int n_pass = (pair && qt_lo != qt_hi) ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    const int qt = pass == 0 ? qt_hi : qt_lo;
    if (pass > 0) __syncthreads();  // every wave is done with the LDS stages before they are refilled
    const int q0 = qt * C::BR;
    // the lane-derived offsets below are recomputed per pass instead of being held (and spilled) across both
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const size_t head_q = (size_t)bh * p.Nq * D;
    int nkv = p.Nkv;  // keys of this (batch, head)
    size_t head_kv = (size_t)bh * p.Nkv * D;
    const int* __restrict__ tab = nullptr;
    if constexpr (PAGED) {  // bh = b * H_kv + h_kv; the head's rows start at h_kv << lg_page inside every page
      const int b = bh / p.Hkv;
      nkv = min(max(p.seq_lens[b], 0), p.max_blocks << p.lg_page);
      head_kv = (size_t)(bh - b * p.Hkv) * ((size_t)D << p.lg_page);
      tab = p.table + (size_t)b * p.max_blocks;
    }
    const uint16_t* __restrict__ qg = p.q + head_q;
    const uint16_t* __restrict__ kg = p.k + head_kv;
    const uint16_t* __restrict__ vg = p.v + head_kv;
    const int qw0 = q0 + w * 32;  // first query row of this wave
    const int qi = qw0 + l32;     // this lane's query row
    const float c = p.c;

    // Q^T fragments: lane holds query qi, d = ks*16 + 8h .. +7.
    bf16x8 qf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi < p.Nq) x = load16(qg + (size_t)qi * D + ks * 16 + 8 * h);
      x ^= p.qxor;
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }

    int kv_end = nkv;
    if (CAUSAL) kv_end = min(nkv, q0 + C::BR + p.off);
    int t_beg = 0, n_tiles = (kv_end + C::BC - 1) / C::BC;  // tiles [t_beg, n_tiles) of this work-group
    if (SPLIT) {
      // a paged sequence's own length is cut into S ranges (lengths are only known on the device)
      const int per = PAGED ? (n_tiles + p.S - 1) / p.S : p.split_tiles;
      t_beg = min(split * per, n_tiles);
      n_tiles = min(t_beg + per, n_tiles);
    }
    // keys this wave needs (0 when the wave's rows lie past N_q)
    const int wave_kv_end = qw0 >= p.Nq ? 0 : (CAUSAL ? min(nkv, qw0 + 32 + p.off) : nkv);
    const int lim = CAUSAL ? min(nkv - 1, qi + p.off) : nkv - 1;  // last key this row may attend

    f32x16 oacc[C::MBD];
#pragma unroll
    for (int mbd = 0; mbd < C::MBD; ++mbd) oacc[mbd] = f32x16{};
    float m_run = kNegInf, l_run = 0.f, lh_run = 0.f;

    // ---------------------------------------------------------------- global -> LDS (direct, no registers)
    // Load i of wave w fills the 1 KB block (w * LPT + i) of a tile: rows RPL*(w*LPT+i) + lane/CH, physical
    // chunk lane%CH, which holds logical chunk (lane%CH) ^ swizzle(row).  The per-lane byte offsets within
    // a tile are fixed; each tile gets a buffer resource starting at its first key and ending at N_kv, so
    // the loads need no vector address arithmetic and rows past N_kv read zeros (their scores are masked).
    int ld_k[C::LPT], ld_v[C::LPT];
#pragma unroll
    for (int i = 0; i < C::LPT; ++i) {
      const int r = C::RPL * (w * C::LPT + i) + lane / C::CH, pc = lane % C::CH;
      ld_k[i] = r * C::ROWB + 16 * (pc ^ swz_k<D>(r));
      ld_v[i] = r * C::ROWB + 16 * (pc ^ swz_v<D>(r));
    }
    // Paged cache: a 1 KB block (RPL rows, RPL <= 8 <= page size, blocks aligned to RPL) never straddles a
    // page, so each block gets a descriptor of its own at its page row, spanning the block's rows that lie
    // before the sequence end, or nothing (zeros land in LDS) when the table entry lies outside the pool.
    // A tile's 64 keys span at most 64 / page size (<= 8) pages: lane i of every wave loads the tile's i-th
    // entry (-1 if outside the pool), one tile ahead of the K / V loads that need it, and the blocks read
    // their entry back with readlane.  absent0/1 hold, per stage, one bit per key of the tile whose entry
    // lies outside the pool; those keys take the masked path and get zero weight, like keys past the end.
    uint64_t absent0 = 0, absent1 = 0;
    int ent_nx = -1;
    auto fetch_entries = [&](int t) {
      if constexpr (PAGED) {
        const int kv0 = t * C::BC, lg = p.lg_page;
        const int pg0 = kv0 >> lg, n_ent = ((min(kv0 + C::BC, nkv) - 1) >> lg) - pg0 + 1;
        int e = -1;
        if (lane < n_ent) e = tab[pg0 + lane];
        ent_nx = (e >= 0 && e < p.num_pages) ? e : -1;
      }
    };
    auto load_tile = [&](int t, int stage) {
      const int kv0 = t * C::BC;
      if constexpr (PAGED) {
        const int lg = p.lg_page, pmask = (1 << lg) - 1;
        const int ent = ent_nx;
        const int n_ent = ((min(kv0 + C::BC, nkv) - 1) >> lg) - (kv0 >> lg) + 1;
        const uint64_t holes = __builtin_amdgcn_ballot_w64(lane < n_ent && ent < 0);
        uint64_t bad = 0;
        if (holes) {
          if (lg >= 6) {
            bad = ~0ull;
          } else {
            const uint64_t page_keys = (1ull << (1 << lg)) - 1;
            for (int i = 0; i < n_ent; ++i)
              if ((holes >> i) & 1) bad |= page_keys << (i << lg);
          }
        }
        if (stage == 0)
          absent0 = bad;
        else
          absent1 = bad;
#pragma unroll
        for (int i = 0; i < C::LPT; ++i) {
          const int rb = C::RPL * (w * C::LPT + i);  // first row of the block within the tile
          const int r0 = kv0 + rb;
          const int e = __builtin_amdgcn_readlane(ent, lg >= 6 ? 0 : rb >> lg);
          int bytes = 0;
          size_t row_el = 0;
          if (r0 < nkv && e >= 0) {
            bytes = min(C::RPL, nkv - r0) * C::ROWB;
            row_el = ((((size_t)e * p.Hkv) << lg) + (r0 & pmask)) * D;
          }
          const int blk = 1024 * (w * C::LPT + i);
          load16_lds(make_rsrc(kg + row_el, bytes), ld_k[i] - rb * C::ROWB, kbuf(stage) + blk);
          load16_lds(make_rsrc(vg + row_el, bytes), ld_v[i] - rb * C::ROWB, vbuf(stage) + blk);
        }
      } else {
        const int bytes = (nkv - kv0) * C::ROWB;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)kv0 * D, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)kv0 * D, bytes);
#pragma unroll
        for (int i = 0; i < C::LPT; ++i) {
          const int blk = 1024 * (w * C::LPT + i);
          load16_lds(rk, ld_k[i], kbuf(stage) + blk);
          load16_lds(rv, ld_v[i], vbuf(stage) + blk);
        }
      }
    };

    // ---------------------------------------------------------------- fragment addresses (bytes)
    // K (A operand of S^T): row 32*mb + l32, logical chunk 2ks + h.
    int k_off[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) k_off[ks] = l32 * C::ROWB + 16 * ((2 * ks + h) ^ swz_k<D>(l32));
    // V^T (A operand of O^T) through ds_read_b64_tr_b16: in lane group G = lane/16 (h = G/2, dh = G%2),
    // lane j points at row key0 + j/4, d = 32*mbd + 16*dh + 4*(j%4); lane i then receives
    // V[key0 + t][32*mbd + 16*dh + i], t = 0..3, with key0 = 16*kc + 8*u + 4*h.  The swizzle of those
    // rows only depends on j/4, so each mbd has one per-lane base and (kc, u) are immediate offsets.
    const int tr_j = lane & 15, tr_dh = (lane >> 4) & 1, tr_row = 4 * h + tr_j / 4;
    int v_off[C::MBD];
#pragma unroll
    for (int mbd = 0; mbd < C::MBD; ++mbd) {
      const int d0 = 32 * mbd + 16 * tr_dh + 4 * (tr_j & 3);
      v_off[mbd] = tr_row * C::ROWB + 16 * ((d0 >> 3) ^ swz_v<D>(tr_row)) + 2 * (d0 & 7);
    }

    // ---------------------------------------------------------------- one tile
    // `next()` issues this wave's loads of the next tile.  It runs right after the S MFMAs are issued, so
    // the data lands in LDS during the softmax, when the wave reads no fragments (direct LDS writes that
    // land during the fragment reads of the MFMA phases slow those reads down).
    auto compute_tile = [&](auto stage_tag, bool masked, int kv0, auto&& next) {
      constexpr int STAGE = decltype(stage_tag)::value;
      const uint8_t* sb = kbuf(STAGE);
      const uint8_t* svb = vbuf(STAGE);
      // S^T = K Q^T for the 64 keys of the tile (two 32-key blocks).  The wave raises its issue
      // priority for its MFMA phases and drops it for the softmax, so when both waves of a SIMD are
      // ready the matrix-core work goes first and the other wave's vector work fills in around it.
      // Decode-like launches (NT: one work-group per key range, few query rows, only wave 0 computes) are
      // bound by the bytes in flight, so the next tile's loads go out first (+2% on grouped-head decode).
      // A paged cache keeps the later point: its loads need the table entries fetched this tile.
      constexpr bool kEarlyLoads = NT && !PAGED;
      if constexpr (kEarlyLoads) next();
      __builtin_amdgcn_s_setprio(1);
      f32x16 S[C::NBLK];
#pragma unroll
      for (int mb = 0; mb < C::NBLK; ++mb) S[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int mb = 0; mb < C::NBLK; ++mb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sb + k_off[ks] + mb * 32 * C::ROWB);
          S[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], S[mb], 0, 0, 0);
        }
      }
      // Keep kKDepth K fragment reads in flight ahead of the MFMAs (left alone, the compiler reads two
      // ahead, and each MFMA pair waits for LDS latency): reads 0..kKDepth-1, then MFMA / read pairs.
      {
        constexpr int NK = C::KS * C::NBLK;
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kKDepth, 0);
#pragma unroll
        for (int i = 0; i < NK - kKDepth; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kKDepth, 0);
      }
      // V^T fragments of the whole tile, read now so their LDS latency passes during the softmax; in
      // prefill launches the next tile's loads go out right after them (+0.7% over the other order)
      bf16x8 vfr[2 * C::NBLK][C::MBD];
#pragma unroll
      for (int kc = 0; kc < 2 * C::NBLK; ++kc)
#pragma unroll
        for (int mbd = 0; mbd < C::MBD; ++mbd) {
          const uint8_t* vb = svb + v_off[mbd] + 16 * kc * C::ROWB;
          const s16x4 lo = lds_read_tr16(vb);
          const s16x4 hi = lds_read_tr16(vb + 8 * C::ROWB);
          vfr[kc][mbd] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!kEarlyLoads) next();
      // mask (diagonal and ragged-tail tiles only; the rest of the tile is one code path)
      if (masked) {
        const int rel = lim - kv0 - 4 * h;  // key offset within the tile allowed iff 8*(r/4) + (r%4) + 32*mb <= rel
        const uint64_t ab = PAGED ? ((STAGE == 0 ? absent0 : absent1) >> (4 * h)) : 0;
#pragma unroll
        for (int mb = 0; mb < C::NBLK; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 32 * mb + 8 * (r >> 2) + (r & 3);
            if (kk > rel || (PAGED && ((ab >> kk) & 1))) S[mb][r] = kNegInf;
          }
      }
      // Online softmax against the running reference maximum m: the weights are 2^(x - m).  Only the
      // first tile of a wave (m = -inf) and tiles whose weights would exceed 2^64 reduce the tile's
      // maximum, move m and rescale O, l; every other tile skips the max reduction (O / l and the LSE do
      // not depend on which reference is used, and 2^64 keeps every sum far from fp32 overflow).
      __builtin_amdgcn_s_setprio(0);
      float rs, rsh;
      bf16x8 P[2 * C::NBLK];
      auto weights = [&](float mref) {
        float part[4] = {0.f, 0.f, 0.f, 0.f};
        rsh = 0.f;
#pragma unroll
        for (int kc = 0; kc < 2 * C::NBLK; ++kc) {
          float pr[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            pr[i] = exp2_hw(fmaf(S[kc >> 1][8 * (kc & 1) + i], c, -mref));
            part[i & 3] += pr[i];
          }
          u32x4 pk;
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(pr[2 * i], pr[2 * i + 1]);
          P[kc] = __builtin_bit_cast(bf16x8, pk);
          rsh = sum_bf16x8(P[kc], rsh);
        }
        rs = (part[0] + part[1]) + (part[2] + part[3]);
      };
      bool slow = __builtin_amdgcn_ballot_w64(m_run == kNegInf) != 0;
      if (!slow) {
        weights(m_run);
        slow = __builtin_amdgcn_ballot_w64(!(rs <= kBig)) != 0;  // also true for inf / nan
      }
      float alpha = 1.f;
      if (slow) {
        float mx = S[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[0][r]);
#pragma unroll
        for (int mb = 1; mb < C::NBLK; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[mb][r]);
        const float mn = fmaxf(m_run, pair_max(mx) * c);
        alpha = (m_run == kNegInf) ? 0.f : exp2_hw(m_run - mn);
        m_run = mn;
        // a row none of whose keys so far is allowed (possible only inside a key range of a split) keeps
        // m = -inf and gets zero weights (reference 0 instead of -inf avoids -inf - (-inf))
        weights(mn == kNegInf ? 0.f : mn);
#pragma unroll
        for (int mbd = 0; mbd < C::MBD; ++mbd) oacc[mbd] *= alpha;
      }
      l_run = alpha * l_run + rs;
      lh_run = alpha * lh_run + rsh;
      // O^T += V^T P^T, one 16-key chunk at a time across the d blocks (independent accumulators back to
      // back, so no MFMA waits for the previous one's result)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kc = 0; kc < 2 * C::NBLK; ++kc) {
#pragma unroll
        for (int mbd = 0; mbd < C::MBD; ++mbd)
          oacc[mbd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[kc][mbd], P[kc], oacc[mbd], 0, 0, 0);
      }
    };

    // One loop iteration per tile: wait for this wave's loads of tile t, barrier (now every wave's loads
    // of tile t have landed and every wave has finished tile t-1, whose stage is reused), start loading
    // tile t+1, compute tile t.  The loop is unrolled by two so each stage index is a compile-time value.
    auto tile = [&](auto stage_tag, int t) {
      constexpr int STAGE = decltype(stage_tag)::value;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const bool more = t + 1 < n_tiles;
      if (PAGED && more) fetch_entries(t + 1);
      auto next = [&]() {
        if (more) load_tile(t + 1, STAGE ^ 1);
      };
      const int kv0 = t * C::BC;
      const bool holes = PAGED && (STAGE == 0 ? absent0 : absent1) != 0;
      if (kv0 < wave_kv_end)
        compute_tile(stage_tag, (kv0 + C::BC > nkv) || (CAUSAL && kv0 + C::BC - 1 > qw0 + p.off) || holes, kv0, next);
      else if (more)
        load_tile(t + 1, STAGE ^ 1);
    };

    // the two stages alternate from the first tile of the range, so stage = (t - t_beg) & 1
    if (t_beg < n_tiles) {
      fetch_entries(t_beg);
      load_tile(t_beg, 0);
    }
    for (int t = t_beg; t < n_tiles; t += 2) {
      tile(std::integral_constant<int, 0>{}, t);
      if (t + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, t + 1);
    }

    // ---------------------------------------------------------------- epilogue
    // O / l_hat (the weights that entered the value product) rounded to bf16, LSE from the fp32 sum.
    const float lt = pair_sum(l_run);
    const float inv = 1.f / pair_sum(lh_run);
    if (SPLIT) {  // fp32 partial of this key range; a row with no key in it gets O = 0, LSE = -inf
      if (qi < p.Nq) {
        const size_t row = (size_t)bh * p.Nq + qi;
        const bool any = lt > 0.f;
        float* orow = p.ws_o + (row * p.S + split) * D;
#pragma unroll
        for (int mbd = 0; mbd < C::MBD; ++mbd)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 val;
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] = any ? oacc[mbd][4 * g4 + e] * inv : 0.f;
            *reinterpret_cast<f32x4*>(orow + mbd * 32 + 8 * g4 + 4 * h) = val;
          }
        if (h == 0) p.ws_lse[row * p.S + split] = any ? (m_run + log2_hw(lt)) * kLn2 : kNegInf;
      }
      return;
    }
    if (qi < p.Nq) {
      uint16_t* orow = p.o + head_q + (size_t)qi * D;
#pragma unroll
      for (int mbd = 0; mbd < C::MBD; ++mbd)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& a = oacc[mbd];
          u32x2 val;
          val[0] = pack_bf16x2(a[4 * g4 + 0] * inv, a[4 * g4 + 1] * inv);
          val[1] = pack_bf16x2(a[4 * g4 + 2] * inv, a[4 * g4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + mbd * 32 + 8 * g4 + 4 * h) = val;
        }
      if (h == 0 && p.lse) p.lse[(size_t)bh * p.Nq + qi] = (m_run + log2_hw(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------------------------- launch

#ifndef FA_PREFILL_D64_UNIT
int64_t prefill_bf16_grid(int B, int H, int Nq, int d, int splits) {
  const int br = 128;  // the smallest query tile of any launch (an upper bound on the grid)
  return (int64_t)B * H * ((Nq + br - 1) / br) * (splits > 0 ? splits : 1);
}
#endif

template <int D, bool CAUSAL, bool SPLIT, bool PAGED = false, bool NT = false, int NW = 4>
hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t s) {
  using C = Cfg<D, NW>;
  PrefillParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.Nq = a.Nq;
  p.Nkv = a.Nkv;
  p.off = a.Nkv - a.Nq;
  p.n_qt = (a.Nq + C::BR - 1) / C::BR;
  p.S = SPLIT ? a.splits : 1;
  p.split_tiles = prefill_split_tiles(a.Nkv, p.S);
  p.total = a.B * a.H * p.n_qt * p.S;
  p.c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-126f);
  p.qxor = a.scale < 0.f ? 0x80008000u : 0u;
  p.ws_o = a.ws_o;
  p.ws_lse = a.ws_lse;
  p.table = a.block_table;
  p.seq_lens = a.seq_lens;
  p.Hkv = a.H;
  p.num_pages = a.num_pages;
  p.max_blocks = a.max_blocks;
  int lg = 0;
  while ((1 << lg) < a.page_size) ++lg;
  p.lg_page = lg;
  // pair causal query tiles when the grid spans at least two work-groups per compute unit (below that
  // every tile runs at once and pairing would only lengthen the longest chain)
  p.pair = CAUSAL && !SPLIT && p.n_qt >= 2 && (int64_t)a.B * a.H * p.n_qt >= 2 * (int64_t)a.num_cu;
  if (p.pair) p.total = a.B * a.H * ((p.n_qt + 1) / 2);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, SPLIT, PAGED, NT, NW>), dim3(p.total), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

#ifndef FA_PREFILL_D64_UNIT
// The d = 64 instances are compiled in their own unit (prefill_bf16_d64.hip), with the scheduler
// strategy that measured fastest for them; this unit only refers to them.
extern template hipError_t launch_prefill_d<64, false, true, true, false, 4>(const PrefillArgs&, hipStream_t);
extern template hipError_t launch_prefill_d<64, false, true, true, true, 4>(const PrefillArgs&, hipStream_t);
extern template hipError_t launch_prefill_d<64, true, true, false, true, 4>(const PrefillArgs&, hipStream_t);
extern template hipError_t launch_prefill_d<64, false, true, false, true, 4>(const PrefillArgs&, hipStream_t);
extern template hipError_t launch_prefill_d<64, true, true, false, false, 4>(const PrefillArgs&, hipStream_t);
extern template hipError_t launch_prefill_d<64, false, true, false, false, 4>(const PrefillArgs&, hipStream_t);
extern template hipError_t launch_prefill_d<64, true, false, false, false, 4>(const PrefillArgs&, hipStream_t);
extern template hipError_t launch_prefill_d<64, false, false, false, false, 4>(const PrefillArgs&, hipStream_t);

LaunchPlan plan_prefill_bf16(int B, int H, int Nq, int d, bool causal, int splits, int num_cu) {
  LaunchPlan pl;
  // d = 128 with at least one 8-wave work-group (256 query rows) per CU: 8 waves, which share each K / V
  // tile between twice the rows (A/B: +0.5-1.1% at B1 H32 N8192, +2.7% at B1 H8 N32768); smaller grids
  // (-18% for 1000 queries x 32 heads, half the CUs idle) and d = 64 (-3.5%) keep 4 waves
  const bool eight = splits == 0 && d == 128 && (int64_t)B * H * ((Nq + 255) / 256) >= num_cu;
  pl.kernel = splits > 0 ? kKernelBf16Split : (eight ? kKernelBf16EightWave : kKernelBf16FourWave);
  pl.waves = eight ? 8 : 4;
  pl.rows = 32 * pl.waves;
  const int n_qt = (Nq + pl.rows - 1) / pl.rows;
  pl.paired = causal && splits == 0 && n_qt >= 2 && (int64_t)B * H * n_qt >= 2 * (int64_t)num_cu;
  pl.groups = (int64_t)B * H * (pl.paired ? (n_qt + 1) / 2 : n_qt) * (splits > 0 ? splits : 1);
  return pl;
}

int prefill_split_tiles(int Nkv, int S) {
  const int tiles = (Nkv + Cfg<128>::BC - 1) / Cfg<128>::BC;
  return (tiles + S - 1) / S;
}

hipError_t launch_prefill_paged_bf16(const PrefillArgs& a, hipStream_t s) {
  if (a.Nq > (a.d == 128 ? Cfg<128>::BR : Cfg<64>::BR))  // more than one query tile re-reads every page
    return a.d == 128 ? launch_prefill_d<128, false, true, true, false>(a, s) : launch_prefill_d<64, false, true, true, false>(a, s);
  return a.d == 128 ? launch_prefill_d<128, false, true, true, true>(a, s) : launch_prefill_d<64, false, true, true, true>(a, s);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  if (a.splits > 0) {
    if (a.Nq <= (a.d == 128 ? Cfg<128>::BR : Cfg<64>::BR)) {  // one query tile: K and V are streamed once
      if (a.d == 128)
        return a.causal ? launch_prefill_d<128, true, true, false, true>(a, s) : launch_prefill_d<128, false, true, false, true>(a, s);
      return a.causal ? launch_prefill_d<64, true, true, false, true>(a, s) : launch_prefill_d<64, false, true, false, true>(a, s);
    }
    if (a.d == 128) return a.causal ? launch_prefill_d<128, true, true>(a, s) : launch_prefill_d<128, false, true>(a, s);
    return a.causal ? launch_prefill_d<64, true, true>(a, s) : launch_prefill_d<64, false, true>(a, s);
  }
  if (plan_prefill_bf16(a.B, a.H, a.Nq, a.d, a.causal, 0, a.num_cu).waves == 8)
    return a.causal ? launch_prefill_d<128, true, false, false, false, 8>(a, s) : launch_prefill_d<128, false, false, false, false, 8>(a, s);
  if (a.d == 128) return a.causal ? launch_prefill_d<128, true, false>(a, s) : launch_prefill_d<128, false, false>(a, s);
  return a.causal ? launch_prefill_d<64, true, false>(a, s) : launch_prefill_d<64, false, false>(a, s);
}

#else
template hipError_t launch_prefill_d<64, false, true, true, false, 4>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prefill_d<64, false, true, true, true, 4>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prefill_d<64, true, true, false, true, 4>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prefill_d<64, false, true, false, true, 4>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prefill_d<64, true, true, false, false, 4>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prefill_d<64, false, true, false, false, 4>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prefill_d<64, true, false, false, false, 4>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prefill_d<64, false, false, false, false, 4>(const PrefillArgs&, hipStream_t);
#endif

}  // namespace fa
