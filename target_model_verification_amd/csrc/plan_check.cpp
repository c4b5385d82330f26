// Host replay of the stream-K walk of the weight-streaming phases (the
// control flow of gemm_phase / next_batch in pass.hip, step for step),
// checking every index the device would form against the buffer sizes the
// host allocates.  Run once per shape by spec_verify_create before the
// first launch, and by the CPU tests over many shapes and grid sizes.
#include <algorithm>
#include <map>
#include <string>
#include <utility>
#include <vector>

#include "stream_plan.h"

namespace sv {
namespace {

struct Batch {
  int u, n, slot, win, sg, c;
};

struct Seg {
  int idx, n, win, c, len, g;
};

std::string at(const GemmShape& s, int n_slots, int g, int G) {
  return std::string(s.name) + " (slots " + std::to_string(n_slots) + ", workgroup " + std::to_string(g) + "/" +
         std::to_string(G) + "): ";
}

}  // namespace

bool check_gemm_walk(const GemmShape& s, int G, size_t ws_floats, size_t n_tickets, std::string& err) {
  const Mat& M = s.M;
  const int U = batch_chunks(s.wf, s.tpu), ACH = a_chunks(s.wf);
  const long long frags = (long long)M.n_sg * M.nkc * kWaves * s.tpu;
  if (M.n_sg >= (1 << 20) || s.max_slots >= (1 << 11)) {
    err = std::string(s.name) + ": too many supergroups or slots for the pending-list encoding";
    return false;
  }
  if (M.w_stride != frags * 1024) {
    err = std::string(s.name) + ": weight stride does not match the fragment count";
    return false;
  }
  const int lo = s.max_slots > 1 ? std::max(1, s.n_shared) : 1;
  for (int n_slots = lo; n_slots <= s.max_slots; ++n_slots) {
    if ((long long)n_slots * M.n_sg * M.nkc >= (1LL << 31)) {
      err = std::string(s.name) + ": phase too large for 32-bit unit indices";
      return false;
    }
    // routed experts take the highest stack indices (the worst case for bounds)
    const int uc = s.max_slots > 1 ? n_slots - s.n_shared : 0;
    std::vector<int> ulist;
    for (int i = 0; i < uc; ++i) ulist.push_back(s.n_experts - uc + i);
    const Lin L = s.max_slots > 1 ? make_lin(M, n_slots, s.slot_major, ulist.data(), uc, s.n_experts)
                                  : make_lin(M, n_slots, s.slot_major);
    std::map<std::pair<int, int>, std::vector<Seg>> segs;     // (slot, sg) -> its segments
    std::map<std::pair<int, int>, int> announced;             // (slot, sg) -> segment count

    for (int g = 0; g < G; ++g) {
      const int u0 = run_begin(L, g, G), u1 = run_begin(L, g + 1, G);
      if (u0 >= u1) continue;
      const std::string where = at(s, n_slots, g, G);
      auto fail = [&](const std::string& m) {
        err = where + m;
        return false;
      };
      // ---- A windows
      auto stage_ok = [&](int key, int win) {
        if (win < 0 || win >= L.n_win || key < 0 || key >= n_slots) return false;
        const long long n16 = (long long)L.wlen(win) * ACH * 128;
        const long long src = (long long)key * s.a_slot + (long long)win * L.W * ACH * 128;
        return n16 * 16 <= kAWindowBytes && src >= 0 && src + n16 <= s.a_size;
      };
      int sk = -1, sw = -1;   // the staged (key, window)
      {
        const Cur a = cur_at(L, u0);
        sk = s.slot_major ? a.slot : 0;
        sw = a.win;
        if (!stage_ok(sk, sw)) return fail("first A window out of bounds");
      }
      // ---- load cursor (the first batch is issued before the phase)
      std::vector<Batch> loads;
      Cur lq = cur_at(L, u0);
      bool ldone = false;
      auto load = [&]() -> bool {
        if (ldone) return true;
        const int n = std::min(U, seg_left(lq, u1));
        if (n < 1) return false;
        if (lq.e < 0 || lq.e >= s.n_stack) return false;
        for (int w = 0; w < kWaves; ++w) {
          if (lq.sg * kWaves + w >= M.n_units) continue;   // idle wave: no loads
          const long long fi0 = (((long long)lq.sg * M.nkc + (long long)lq.win * M.win + lq.c) * kWaves + w) * s.tpu;
          for (int i = 0; i < n; ++i) {   // slots past n are zero-filled
            for (int t = 0; t < s.tpu; ++t) {
              const long long fi = fi0 + (long long)i * kWaves * s.tpu + t;
              if (fi < 0 || fi >= frags) return false;
            }
          }
        }
        loads.push_back({lq.u, n, lq.slot, lq.win, lq.sg, lq.c});
        batch_advance(L, lq, n, u1, ldone);
        return true;
      };
      if (!load()) return fail("first weight batch out of bounds");
      // ---- compute cursor
      Cur cc = cur_at(L, u0);
      int pend = 0;
      size_t next = 0;
      for (;;) {
        const int nch = seg_left(cc, u1);
        if (nch < 1) return fail("empty segment");
        const int key = s.slot_major ? cc.slot : 0;
        if (key != sk || cc.win != sw) return fail("segment computed against a different A window");
        for (int c0 = 0; c0 < nch; c0 += U) {
          const int n = std::min(U, nch - c0);
          if ((cc.c + c0 + n) > L.wlen(cc.win)) return fail("A chunk past the staged window");
          if (next >= loads.size()) return fail("compute ahead of the loads");
          const Batch& b = loads[next++];
          if (b.u != cc.u + c0 || b.n != n || b.slot != cc.slot || b.win != cc.win || b.sg != cc.sg ||
              b.c != cc.c + c0)
            return fail("loaded batch differs from the computed one");
          if (!load()) return fail("weight batch out of bounds");
        }
        const int c_start = cc.c;
        cc.u += nch;
        cc.c += nch;
        int idx = 0, nseg = 0;
        if (s.fixed) seg_info_fixed(L, cc.slot, cc.sg, cc.win, g, G, idx, nseg);
        else seg_info(L, cc.slot, cc.sg, cc.win, g, G, idx, nseg);
        // partials this segment hands over: one, or (fixed order, a segment
        // after the block's first) one per piece, i.e. per batch
        const int nparts = s.fixed && idx > 0 ? (nch + U - 1) / U : 1;
        if (nseg < 1 || nseg > M.max_seg || idx < 0 || idx + nparts > nseg) return fail("segment index out of range");
        const std::pair<int, int> blk(cc.slot, cc.sg);
        auto an = announced.find(blk);
        if (an == announced.end()) announced[blk] = nseg;
        else if (an->second != nseg) return fail("segment count differs between workgroups");
        for (int b = 0; b < nparts; ++b) {
          const int c = nparts == 1 ? c_start : c_start + b * U;
          const int len = nparts == 1 ? nch : std::min(U, nch - b * U);
          segs[blk].push_back({idx + b, nseg, cc.win, c, len, g});
          if (nseg > 1) {
            const long long last = (((((long long)cc.slot * M.n_sg + cc.sg) * M.max_seg + idx + b) * kWaves + kWaves - 1) *
                                        s.tpu * 256) + (long long)(s.tpu - 1) * 256 + 63 * 4 + 4;
            if (last > (long long)ws_floats) return fail("split-K partial past the workspace");
            if ((long long)cc.slot * M.n_sg + cc.sg >= (long long)n_tickets) return fail("ticket out of range");
          }
          // every partial may be listed (split ones, and finished blocks of
          // phases that announce their outputs)
          if (++pend > kMaxPending) return fail("too many segments for one workgroup's list");
        }
        if (cc.u >= u1) break;
        seg_advance(L, cc);
        const int nkey = s.slot_major ? cc.slot : 0;
        if (nkey != sk || cc.win != sw) {   // restage
          sk = nkey;
          sw = cc.win;
          if (!stage_ok(sk, sw)) return fail("restaged A window out of bounds");
        }
      }
      if (next != loads.size() || !ldone) return fail("loads left over at the end of the range");
      if (lq.u != u1) return fail("load cursor did not stop at the range end");
    }
    // ---- split-K invariants over all workgroups
    if ((long long)segs.size() != (long long)n_slots * M.n_sg) {
      err = std::string(s.name) + ": not every unit block was computed";
      return false;
    }
    for (auto& kv : segs) {
      std::vector<Seg>& v = kv.second;
      const int n = v.front().n;
      if ((int)v.size() != n) {
        err = std::string(s.name) + ": a unit block has " + std::to_string(v.size()) + " segments, announced " +
              std::to_string(n);
        return false;
      }
      std::sort(v.begin(), v.end(), [](const Seg& a, const Seg& b) { return a.idx < b.idx; });
      int k = 0;   // next K chunk expected
      for (int i = 0; i < n; ++i) {
        const Seg& q = v[i];
        if (q.idx != i || q.win * M.win + q.c != k) {
          err = std::string(s.name) + ": split-K segments out of K order or not covering K";
          return false;
        }
        // fixed order: every partial after the first is one piece (aligned,
        // at most one batch), so the sum does not depend on the work split
        if (s.fixed && i > 0 && (q.len > U || q.c % U != 0)) {
          err = std::string(s.name) + ": a fixed-order partial after the first is not one piece";
          return false;
        }
        k += q.len;
      }
      if (k != M.nkc) {
        err = std::string(s.name) + ": segments of a unit block do not cover K";
        return false;
      }
    }
  }
  return true;
}

}  // namespace sv
