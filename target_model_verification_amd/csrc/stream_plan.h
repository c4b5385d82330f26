// Stream-K planning of the weight-streaming phases, shared by the device
// code (which walks it) and the host runtime (which sizes the split-K
// workspace from it and checks every workgroup's walk before the first
// launch).
//
// A phase over n_slots slots (experts) of one matrix is a flat space of
// units (slot, window, supergroup, chunk).  Each (slot, window, supergroup)
// run of chunks is cut into pieces of U chunks (one weight batch of a wave;
// the last piece of a run may be shorter), and workgroup g of G owns the
// pieces [floor(P g / G), floor(P (g+1) / G)) of the P pieces: every
// workgroup's share starts and ends on a batch boundary, so it streams in
// the fewest batches its share allows (cutting the flat space into equal
// runs of chunks instead leaves partial batches at segment ends, and the
// workgroups with more of them stream longer).  A "segment" is the part of
// one (slot, window, supergroup) run that one workgroup owns; a unit block
// (slot, supergroup) whose K range is split over several segments is
// reduced in K order by a fixed reducer.
#pragma once
#include "sv_common.h"

#if defined(__HIP__)
#define SP_HD __host__ __device__ __forceinline__
#else
#define SP_HD inline
#endif

namespace sv {

SP_HD int sp_min(int a, int b) { return a < b ? a : b; }

// With slot_major the order is (slot, win, sg, c) -- used when A depends on
// the slot (expert down projections); otherwise (win, slot, sg, c), so a
// staged A window serves every slot.
struct Lin {
  int n_slots, n_sg, nkc, W, n_win;
  bool slot_major;
  int total;          // units in the phase (fits in 32 bits for every supported shape)
  int U, npW, npL;    // chunks per piece; pieces per run of a full / of the last window
  int P;              // pieces in the phase
  const int* ulist;   // MoE: routed experts of the pass in slot order (null: dense phase)
  int uc, n_experts;
  // expert (stack index) of a slot: routed experts first, then the shared ones
  SP_HD int expert(int slot) const {
    return ulist ? (slot < uc ? ulist[slot] : n_experts + (slot - uc)) : 0;
  }
  SP_HD int wlen(int win) const { return sp_min(W, nkc - win * W); }
  SP_HD int block_start(int slot, int win) const {
    if (slot_major) return slot * n_sg * nkc + n_sg * W * win;
    return n_slots * n_sg * W * win + slot * n_sg * wlen(win);
  }
  SP_HD int np(int win) const { return win == n_win - 1 ? npL : npW; }
  // first piece of the run (slot, win, supergroup 0)
  SP_HD int piece_start(int slot, int win) const {
    if (slot_major) return slot * n_sg * ((n_win - 1) * npW + npL) + n_sg * npW * win;
    return n_slots * n_sg * npW * win + slot * n_sg * np(win);
  }
  // first chunk of piece p (total for p = P)
  SP_HD int piece_chunk(int p) const {
    if (p >= P) return total;
    int slot, win, r;
    if (slot_major) {
      const int per_slot = n_sg * ((n_win - 1) * npW + npL);
      slot = p / per_slot;
      r = p - slot * per_slot;
      win = r / (n_sg * npW);
      if (win > n_win - 1) win = n_win - 1;
      r -= n_sg * npW * win;
    } else {
      const int per_win = n_slots * n_sg * npW;
      win = p / per_win;
      if (win > n_win - 1) win = n_win - 1;
      r = p - per_win * win;
      const int per_slot = n_sg * np(win);
      slot = r / per_slot;
      r -= slot * per_slot;
    }
    const int sg = r / np(win), q = r - sg * np(win);
    return block_start(slot, win) + sg * wlen(win) + q * U;
  }
};

SP_HD Lin make_lin(const Mat& M, int n_slots, bool slot_major, const int* ulist = nullptr, int uc = 0,
                   int n_experts = 0) {
  Lin L;
  L.ulist = ulist;
  L.uc = uc;
  L.n_experts = n_experts;
  L.n_slots = n_slots;
  L.n_sg = M.n_sg;
  L.nkc = M.nkc;
  L.W = M.win;
  L.n_win = M.n_win;
  L.slot_major = slot_major;
  L.total = n_slots * M.n_sg * M.nkc;
  L.U = M.U;
  L.npW = (L.W + L.U - 1) / L.U;
  L.npL = (L.wlen(L.n_win - 1) + L.U - 1) / L.U;
  L.P = n_slots * M.n_sg * ((L.n_win - 1) * L.npW + L.npL);
  return L;
}

// floor(p / q) for 0 <= p < 2^52 and 0 < q < 2^31.  The device evaluates
// it in double precision: p and q are exact, the quotient is correctly
// rounded with an error of at most (p / q) 2^-53 < 1 / (2q), and a
// non-integral p / q lies at least 1 / q from either neighbouring integer,
// so the floor is the integer quotient.  (A 64-bit integer division is a
// long serial sequence of scalar instructions on the GPU.)
SP_HD int floor_div(long long p, long long q) {
#if defined(__HIP_DEVICE_COMPILE__)
  return (int)floor((double)p / (double)q);
#else
  return (int)(p / q);
#endif
}

// First unit of workgroup g.
SP_HD int range_begin(int total, int g, int G) { return floor_div((long long)total * g, G); }

// Workgroup owning unit u (the largest g with range_begin(g) <= u).
SP_HD int wg_of(int u, int T, int G) { return floor_div(((long long)u + 1) * G - 1, T); }

// First chunk of workgroup g's share (run_begin(L, G, G) = L.total).
SP_HD int run_begin(const Lin& L, int g, int G) { return L.piece_chunk(range_begin(L.P, g, G)); }

// Position in the flattened space (advanced a segment at a time without
// divisions).
struct Cur {
  int u;
  int slot, win, sg, c, len, e;
};

SP_HD Cur cur_at(const Lin& L, int u) {
  Cur q;
  q.u = u;
  if (L.slot_major) {
    const int per_slot = L.n_sg * L.nkc;
    q.slot = u / per_slot;
    int r = u - q.slot * per_slot;
    q.win = sp_min(r / (L.n_sg * L.W), L.n_win - 1);
    r -= L.n_sg * L.W * q.win;
    q.len = L.wlen(q.win);
    q.sg = r / q.len;
    q.c = r - q.sg * q.len;
  } else {
    const int per_win = L.n_slots * L.n_sg * L.W;
    q.win = sp_min(u / per_win, L.n_win - 1);
    int r = u - per_win * q.win;
    q.len = L.wlen(q.win);
    q.slot = r / (L.n_sg * q.len);
    r -= q.slot * L.n_sg * q.len;
    q.sg = r / q.len;
    q.c = r - q.sg * q.len;
  }
  q.e = L.expert(q.slot);
  return q;
}

// Split-K bookkeeping of unit block (slot, sg): number of segments over all
// windows and workgroups, and the index of the segment (win, g) in K order.
// With at least as many pieces as workgroups every workgroup owns a
// non-empty share, so the workgroups covering a run are consecutive; with
// fewer, each owns at most one piece and a piece's owner is unique.
SP_HD void seg_info(const Lin& L, int slot, int sg, int win, int g, int G, int& idx, int& n) {
  n = 0;
  idx = 0;
  const bool sparse = L.P < G;
  for (int w = 0; w < L.n_win; ++w) {
    const int a = L.piece_start(slot, w) + sg * L.np(w);
    const int b = a + L.np(w) - 1;
    if (sparse) {
      if (w == win) idx = n + (range_begin(L.P, g, G) - a);
      n += L.np(w);
    } else {
      const int ga = wg_of(a, L.P, G), gb = wg_of(b, L.P, G);
      if (w == win) idx = n + (g - ga);
      n += gb - ga + 1;
    }
  }
}

// Split-K bookkeeping in a fixed summation order (expert phases, whose
// slot count, and with it the work split, follows the routed union): the
// value of unit block (slot, sg) is the chain (((P_0 + P_1) + P_2) + ...)
// over its pieces in K order, each piece summed from zero, whichever
// workgroups own them.  The segment holding the block's first piece hands
// over its own chain as partial 0; every piece of a later segment is a
// partial of its own.  n: partials of the block; idx: partial index of the
// first piece of segment (win, g) (0 when it holds the block's first piece).
SP_HD void seg_info_fixed(const Lin& L, int slot, int sg, int win, int g, int G, int& idx, int& n) {
  const bool sparse = L.P < G;
  const int a0 = L.piece_start(slot, 0) + sg * L.np(0);
  // pieces of the first segment: those of window 0's run owned by the owner
  // of its first piece (one piece each when pieces are scarcer than workgroups)
  const int f = sparse ? 1 : sp_min(L.np(0), range_begin(L.P, wg_of(a0, L.P, G) + 1, G) - a0);
  int tot = 0, j = 0;
  const int mine = range_begin(L.P, g, G);
  for (int w = 0; w < L.n_win; ++w) {
    if (w == win) {
      const int a = L.piece_start(slot, w) + sg * L.np(w);
      j = tot + (mine > a ? mine - a : 0);
    }
    tot += L.np(w);
  }
  n = tot - f + 1;
  idx = j == 0 ? 0 : j - f + 1;
}

// Units left in the cursor's current segment, capped by the range end.
SP_HD int seg_left(const Cur& q, int u1) { return sp_min(q.len - q.c, u1 - q.u); }

// Moves a cursor that reached the end of its segment to the next segment.
SP_HD void seg_advance(const Lin& L, Cur& q) {
  q.c = 0;
  if (++q.sg < L.n_sg) return;
  q.sg = 0;
  if (L.slot_major) {
    if (++q.win == L.n_win) { q.win = 0; ++q.slot; q.e = L.expert(q.slot); }
  } else {
    if (++q.slot == L.n_slots) { q.slot = 0; ++q.win; }
    q.e = L.expert(q.slot);
  }
  q.len = (q.win < L.n_win) ? L.wlen(q.win) : 1;
}

// Moves a cursor past one batch of n chunks of its segment; sets done at
// the range end, else steps into the next segment when this one is used up.
SP_HD void batch_advance(const Lin& L, Cur& q, int n, int u1, bool& done) {
  q.u += n;
  q.c += n;
  if (q.c == q.len || q.u >= u1) {
    if (q.u >= u1) done = true;
    else seg_advance(L, q);
  }
}

// Chunks per weight batch of one wave: a ring of kRing 16-byte registers
// per lane (1 KB fragments), two per fp32 chunk (hi and lo); int4 batches
// use half the ring, since each int4 register expands to four bf16 ones
// while it is consumed.
SP_HD constexpr int batch_chunks(int wf, int tpu) {
  return wf == W_INT4 ? kRing / (2 * tpu) : kRing / (tpu * (wf == W_F32 ? 2 : 1));
}

// 32-k A-operand chunks per weight chunk.
SP_HD constexpr int a_chunks(int wf) { return wf == W_INT4 ? 4 : 1; }

// ------------------------------------------------------------------ host side
}  // namespace sv
#include <string>
namespace sv {

// Streaming geometry of a matrix of K x N (n_units output units of tpu
// tiles each); window_k bounds the K elements of one staged A window.
inline void mat_geometry(Mat& M, int wf, int K, int N, int n_units, int tpu, int window_k) {
  M.K = K;
  M.N = N;
  M.n_units = n_units;
  M.n_sg = (n_units + kWaves - 1) / kWaves;
  const int chunk_k = wf == W_INT4 ? kGroupK : kChunkK;
  M.nkc = (K + chunk_k - 1) / chunk_k;
  const int a_win_k = kAWindowBytes / 2048 * kChunkK;   // 2 KB of A per 32 k
  int max_w = (window_k < a_win_k ? window_k : a_win_k) / chunk_k;
  if (max_w < 1) max_w = 1;
  M.n_win = (M.nkc + max_w - 1) / max_w;
  M.win = (M.nkc + M.n_win - 1) / M.n_win;
  const long long frags = (long long)M.n_sg * M.nkc * kWaves * tpu;
  M.w_stride = frags * 1024;
  M.w2_stride = wf == W_INT4 ? frags * 32 : (wf == W_F32 ? M.w_stride : 0);
  M.max_seg = 1;
  M.U = batch_chunks(wf, tpu);
}

// Largest number of split-K partials of one unit block, and the largest
// number of partials one workgroup flushes, for n_slots slots (fixed: the
// fixed-order split of the expert phases).
inline void seg_bounds(const Mat& M, int n_slots, bool slot_major, bool fixed, int G, int& max_seg, int& max_pend) {
  const Lin L = make_lin(M, n_slots, slot_major);
  max_seg = 1;
  for (int s = 0; s < n_slots; ++s)
    for (int sg = 0; sg < M.n_sg; ++sg) {
      int idx = 0, n = 0;
      if (fixed) seg_info_fixed(L, s, sg, 0, 0, G, idx, n);
      else seg_info(L, s, sg, 0, 0, G, idx, n);
      if (n > max_seg) max_seg = n;
    }
  // a share of at most ceil(P / G) pieces meets at most that many runs (and
  // flushes at most one partial per piece)
  max_pend = (int)(((long long)L.P + G - 1) / G) + 2;
}

// One weight-streaming phase shape of a pass, with what its walk may touch.
struct GemmShape {
  const char* name;
  Mat M;               // geometry, M.max_seg included
  int wf, tpu;
  int n_stack;         // matrices stacked (experts); 1 for dense phases
  int n_experts, n_shared;
  int max_slots;       // slots per pass: 1, or routed + shared experts
  bool slot_major;
  bool fixed;          // fixed-order split-K (seg_info_fixed): expert phases
  long long a_slot;    // A operand uint4 per slot (0: one A shared by all slots)
  long long a_size;    // A operand buffer size (uint4)
};

// Replays, on the host, the walk every workgroup of a grid of G makes over
// the phase for every slot count it can see, and checks each weight
// fragment, A window, split-K workspace slot, ticket and pending entry
// against the buffer sizes, plus the split-K invariants (each split unit
// block has exactly its announced number of segments, their indices are
// 0..n-1 in K order and together cover K once).  Returns false with a
// message on the first violation.
bool check_gemm_walk(const GemmShape& s, int G, size_t ws_floats, size_t n_tickets, std::string& err);

}  // namespace sv
