// Plan builder: the ordered stream/event operations of one looped call.
//
// Wang et al., "Overlap Communication with Dependent Computation via
// Decomposition in Large Deep Learning Models" (ASPLOS'23):
//   * Section 5.1 -- the loop, the {source, destination} pairs of its
//     CollectivePermute (rank r sends to r - 1) and the shard movement
//     (AllGather aligned with the partition ID at loop start, ReduceScatter at
//     loop end);
//   * Section 5.2 -- each permute split into a Start that only launches the
//     transfer and a Done that marks its completion: here a copy enqueued on
//     the copy stream followed by an event record (Start), and an event wait
//     on the compute stream right before the first GEMM that reads the data
//     (Done);
//   * Section 5.4.1 -- unrolling by two: the AllGather alternates two receive
//     buffers per rank (no loop-carried alias copy), and the ReduceScatter
//     accumulation chain is split into two interleaved chains so that the
//     transfer of one chain overlaps the fused GEMM+add of the other.
//
// The permute in the last AllGather iteration and the first ReduceScatter
// permute (which would move the zero-initialised accumulator) move nothing
// that is used, so N-1 transfers per rank are built; the first ReduceScatter
// partial is stored instead of added to zero.
//
// Host order matters for events: a wait enqueued before the matching record
// would not wait, so every record below is enqueued before its wait.

#include <cstdio>
#include <string>

#include "cce_internal.hpp"

namespace cce {

namespace {

BufRef ref(uint8_t kind, int rank, int parity = 0, int half = 0) {
  BufRef b;
  b.kind = kind;
  b.rank = static_cast<int16_t>(rank);
  b.parity = static_cast<uint8_t>(parity);
  b.half = static_cast<uint8_t>(half);
  return b;
}

Op rec(StreamId s, int ev) {
  Op o;
  o.kind = OP_RECORD;
  o.stream = s;
  o.event = ev;
  return o;
}

Op wait(StreamId s, int ev) {
  Op o;
  o.kind = OP_WAIT;
  o.stream = s;
  o.event = ev;
  return o;
}

Op hint_wait(StreamId s, int ev) {
  Op o = wait(s, ev);
  o.hint = true;
  return o;
}

}  // namespace

Plan build_allgather_plan(int n, int mode, bool case2_ws, bool serial, bool fused) {
  Plan p;
  p.kind = 0;
  p.n = n;
  p.mode = mode;
  p.serial = serial || fused;
  p.fused = fused;
  serial = p.serial;
  const bool case2 = (mode == CCE_AG_LHS_COLS || mode == CCE_AG_RHS_ROWS);
  // events: 0 fork, 2+i gemm_done[i], 2+n+i arrive[i], 2+2n+i started[i]
  p.n_events = 2 + 3 * n;
  const int EV_FORK = 0;
  auto ev_gemm = [&](int i) { return 2 + i; };
  auto ev_arrive = [&](int i) { return 2 + n + i; };
  auto ev_started = [&](int i) { return 2 + 2 * n + i; };
  const StreamId cs = serial ? S_COMPUTE : S_COPY;

  auto held = [&](int r, int i) {
    return i == 0 ? ref(B_LOOPED, r) : ref(B_RECV, r, i % 2);
  };

  if (!serial && n > 1) {
    p.ops.push_back(rec(S_COMPUTE, EV_FORK));
    p.ops.push_back(wait(S_COPY, EV_FORK));
  }
  for (int i = 0; i < n; ++i) {
    // Start of the permute that brings the shard of iteration i+1 (in the
    // fused form the GEMM of iteration i forwards its shard itself).
    if (i + 1 < n && !fused) {
      // WAR: the destination parity was last read by GEMM(i-1); GEMM(0)
      // reads the caller's shards, so the first two copies need no wait.
      if (!serial && i >= 2) p.ops.push_back(wait(S_COPY, ev_gemm(i - 1)));
      // Mark that the copy stream reached this permute; GEMM(i) waits for
      // the mark, so the copies are dispatched before the GEMM that runs
      // beside them and are not starved of compute units by it.
      if (!serial) p.ops.push_back(rec(S_COPY, ev_started(i)));
      Op c;
      c.kind = OP_COPY;
      c.stream = cs;
      c.iter = i;
      for (int r = 0; r < n; ++r) {
        Item it;
        it.rank = r;
        it.shard = ag_shard(n, r, i + 1);
        it.a = held((r + 1) % n, i);
        it.c = ref(B_RECV, r, (i + 1) % 2);
        c.items.push_back(it);
      }
      p.ops.push_back(c);
      if (!serial) p.ops.push_back(rec(S_COPY, ev_arrive(i + 1)));
    }
    // Done of the permute that brought this iteration's shard, then the GEMM.
    if (!serial && i >= 1) p.ops.push_back(wait(S_COMPUTE, ev_arrive(i)));
    if (!serial && i + 1 < n) p.ops.push_back(hint_wait(S_COMPUTE, ev_started(i)));
    Op g;
    g.kind = OP_GEMM;
    g.stream = S_COMPUTE;
    g.iter = i;
    const bool last = (i == n - 1);
    if (!case2) {
      g.epi = EPI_STORE;
      g.final_store = true;
    } else {
      g.epi = (i == 0) ? EPI_STORE : EPI_ACCUM;
      g.final_store = last || !case2_ws;   // fp32 out accumulates in place
    }
    for (int r = 0; r < n; ++r) {
      Item it;
      it.rank = r;
      it.shard = ag_shard(n, r, i);
      it.a = held(r, i);
      it.b = ref(B_LOCAL, r);
      if (fused && i + 1 < n) {
        it.fwd = ref(B_RECV, (r - 1 + n) % n, (i + 1) % 2);
        it.has_fwd = true;
      }
      const BufRef acc = case2_ws ? ref(B_CASE2, r) : ref(B_OUT, r);
      if (!case2) {
        it.c = ref(B_OUT, r);
      } else {
        it.c = last ? ref(B_OUT, r) : acc;
        if (i > 0) {
          it.cin = acc;
          it.has_cin = true;
        }
      }
      g.items.push_back(it);
    }
    p.ops.push_back(g);
    if (!serial && i >= 1 && i + 2 < n) p.ops.push_back(rec(S_COMPUTE, ev_gemm(i)));
  }
  // No join is needed: the last copy's arrival is waited for by the last
  // GEMM, so all copy-stream work is ordered before later work on `stream`.
  return p;
}

Plan build_reducescatter_plan(int n, int mode, bool two_halves, bool serial, bool fused) {
  Plan p;
  p.kind = 1;
  p.n = n;
  p.mode = mode;
  p.serial = serial || fused;
  p.fused = fused;
  serial = p.serial;
  // Fused: the accumulate epilogue stores into the next rank's accumulator,
  // so there is no copy to overlap and no need for two chains.
  const int H = (two_halves && !fused) ? 2 : 1;
  // events: 2+(2i+h) gemm_done, 2+2n+(2i+h) arrive, 2+4n+(2i+h) started
  p.n_events = 2 + 6 * n;
  auto ev_gemm = [&](int i, int h) { return 2 + 2 * i + h; };
  auto ev_arrive = [&](int i, int h) { return 2 + 2 * n + 2 * i + h; };
  auto ev_started = [&](int i, int h) { return 2 + 4 * n + 2 * i + h; };
  const StreamId cs = serial ? S_COMPUTE : S_COPY;
  // The GEMM that runs beside half-copy (i, h) is the next half-step's.
  auto prev_copy = [&](int i, int h, int* pi, int* ph) {
    if (h == 1) { *pi = i; *ph = 0; } else { *pi = i - 1; *ph = H - 1; }
    return *pi >= 0 && *pi + 1 < n;
  };

  // No fork is needed either: the first copy waits for GEMM(0, 0), which is
  // ordered after the caller's earlier work on `stream`.
  for (int i = 0; i < n; ++i) {
    const bool last = (i == n - 1);
    for (int h = 0; h < H; ++h) {
      if (!serial && i >= 1) p.ops.push_back(wait(S_COMPUTE, ev_arrive(i, h)));
      int pi, ph;
      if (!serial && prev_copy(i, h, &pi, &ph)) p.ops.push_back(hint_wait(S_COMPUTE, ev_started(pi, ph)));
      Op g;
      g.kind = OP_GEMM;
      g.stream = S_COMPUTE;
      g.iter = i;
      g.half = h;
      g.epi = (i == 0) ? EPI_STORE : EPI_ACCUM;
      g.final_store = last;
      for (int r = 0; r < n; ++r) {
        Item it;
        it.rank = r;
        it.shard = rs_slice(n, r, i);
        it.a = ref(B_A, r);
        it.b = ref(B_B, r);
        const BufRef acc = ref(B_ACC, r, i % 2, h);
        // fused: send the new accumulator straight to rank r - 1
        const BufRef dst = fused ? ref(B_ACC, (r - 1 + n) % n, (i + 1) % 2, h) : acc;
        it.c = last ? ref(B_OUT, r, 0, h) : dst;
        if (i > 0) {
          it.cin = acc;   // the accumulator received from rank r + 1
          it.has_cin = true;
        }
        g.items.push_back(it);
      }
      p.ops.push_back(g);
      if (!last && !fused) {
        if (!serial) {
          p.ops.push_back(rec(S_COMPUTE, ev_gemm(i, h)));
          p.ops.push_back(wait(S_COPY, ev_gemm(i, h)));
          p.ops.push_back(rec(S_COPY, ev_started(i, h)));
        }
        Op c;
        c.kind = OP_COPY;
        c.stream = cs;
        c.iter = i;
        c.half = h;
        for (int r = 0; r < n; ++r) {
          Item it;
          it.rank = r;
          it.shard = rs_slice(n, (r + 1) % n, i);
          it.a = ref(B_ACC, (r + 1) % n, i % 2, h);
          it.c = ref(B_ACC, r, (i + 1) % 2, h);
          c.items.push_back(it);
        }
        p.ops.push_back(c);
        if (!serial) p.ops.push_back(rec(S_COPY, ev_arrive(i + 1, h)));
      }
    }
  }
  // No join is needed: the last copy's arrival is waited for by the last
  // GEMM, so all copy-stream work is ordered before later work on `stream`.
  return p;
}

// ---------------------------------------------------------------------------
// Bidirectional transfer ([OV] Section 5.4.2): two partial einsums per
// iteration, one per direction round the ring, in one GEMM launch (2n
// groups), so the loop has ceil(n/2) iterations.  Every rank still sends
// n-1 shards.  The AllGather's counter-clockwise buffer is filled by a
// prologue permute before the loop; the ReduceScatter's counter-clockwise
// accumulator takes one epilogue permute after its last partial, and an
// align-and-sum adds the two accumulators of each shard.
// ---------------------------------------------------------------------------
Plan build_allgather_plan_bidir(int n, int mode, bool serial, bool fused) {
  Plan p;
  p.kind = 0;
  p.n = n;
  p.mode = mode;
  p.serial = serial || fused;
  p.fused = fused;
  p.bidir = true;
  serial = p.serial;
  const int KC = bidir_cw_len(n), KW = bidir_ccw_len(n);
  // events: 0 fork, 1 prologue arrival, 2+i gemm_done[i], 2+n+i arrive[i],
  // 2+2n+i started[i]
  p.n_events = 2 + 3 * n;
  const int EV_FORK = 0, EV_PRO = 1;
  auto ev_gemm = [&](int i) { return 2 + i; };
  auto ev_arrive = [&](int i) { return 2 + n + i; };
  auto ev_started = [&](int i) { return 2 + 2 * n + i; };
  const StreamId cs = serial ? S_COMPUTE : S_COPY;
  auto held_cw = [&](int r, int i) {
    return i == 0 ? ref(B_LOOPED, r) : ref(B_RECV, r, i % 2);
  };
  auto held_ccw = [&](int r, int i) { return ref(B_RECV_CCW, r, i % 2); };
  // The copy op of iteration i brings the shards of iteration i+1.
  auto cw_copy = [&](int i) { return i + 1 < KC; };
  auto ccw_copy = [&](int i) { return i + 1 < KW; };
  // WAR: its destinations were last read by GEMM(i-1) -- the cw parity from
  // iteration 2 on (GEMM(0) reads the caller's shard), the ccw parity from
  // iteration 1 on (GEMM(0) reads the prologue's buffer).
  auto copy_waits = [&](int i) { return (cw_copy(i) && i >= 2) || (ccw_copy(i) && i >= 1); };

  if (!serial && n > 1) {
    p.ops.push_back(rec(S_COMPUTE, EV_FORK));
    p.ops.push_back(wait(S_COPY, EV_FORK));
  }
  if (KW > 0) {            // prologue: rank r's ccw buffer gets rank r-1's shard
    Op c;
    c.kind = OP_COPY;
    c.stream = cs;
    c.iter = -1;
    for (int r = 0; r < n; ++r) {
      Item it;
      it.rank = r;
      it.shard = ag_shard_ccw(n, r, 0);
      it.a = ref(B_LOOPED, mod_n(r - 1, n));
      it.c = ref(B_RECV_CCW, r, 0);
      c.items.push_back(it);
    }
    p.ops.push_back(c);
    if (!serial) p.ops.push_back(rec(S_COPY, EV_PRO));
  }
  for (int i = 0; i < KC; ++i) {
    if (cw_copy(i) && !fused) {
      if (!serial && copy_waits(i)) p.ops.push_back(wait(S_COPY, ev_gemm(i - 1)));
      if (!serial) p.ops.push_back(rec(S_COPY, ev_started(i)));
      Op c;
      c.kind = OP_COPY;
      c.stream = cs;
      c.iter = i;
      for (int r = 0; r < n; ++r) {
        Item it;
        it.rank = r;
        it.shard = ag_shard_cw(n, r, i + 1);
        it.a = held_cw(mod_n(r + 1, n), i);
        it.c = ref(B_RECV, r, (i + 1) % 2);
        c.items.push_back(it);
      }
      if (ccw_copy(i)) {
        for (int r = 0; r < n; ++r) {
          Item it;
          it.rank = r;
          it.shard = ag_shard_ccw(n, r, i + 1);
          it.a = held_ccw(mod_n(r - 1, n), i);
          it.c = ref(B_RECV_CCW, r, (i + 1) % 2);
          c.items.push_back(it);
        }
      }
      p.ops.push_back(c);
      if (!serial) p.ops.push_back(rec(S_COPY, ev_arrive(i + 1)));
    }
    if (!serial) {
      if (i == 0 && KW > 0) p.ops.push_back(wait(S_COMPUTE, EV_PRO));
      if (i >= 1) p.ops.push_back(wait(S_COMPUTE, ev_arrive(i)));
      if (cw_copy(i)) p.ops.push_back(hint_wait(S_COMPUTE, ev_started(i)));
    }
    Op g;
    g.kind = OP_GEMM;
    g.stream = S_COMPUTE;
    g.iter = i;
    g.epi = EPI_STORE;
    g.final_store = true;
    for (int r = 0; r < n; ++r) {
      Item it;
      it.rank = r;
      it.shard = ag_shard_cw(n, r, i);
      it.a = held_cw(r, i);
      it.b = ref(B_LOCAL, r);
      it.c = ref(B_OUT, r);
      if (fused && cw_copy(i)) {
        it.fwd = ref(B_RECV, mod_n(r - 1, n), (i + 1) % 2);
        it.has_fwd = true;
      }
      g.items.push_back(it);
    }
    if (i < KW) {
      for (int r = 0; r < n; ++r) {
        Item it;
        it.rank = r;
        it.shard = ag_shard_ccw(n, r, i);
        it.a = held_ccw(r, i);
        it.b = ref(B_LOCAL, r);
        it.c = ref(B_OUT, r);
        if (fused && ccw_copy(i)) {
          it.fwd = ref(B_RECV_CCW, mod_n(r + 1, n), (i + 1) % 2);
          it.has_fwd = true;
        }
        g.items.push_back(it);
      }
    }
    p.ops.push_back(g);
    if (!serial && i + 1 < KC && copy_waits(i + 1)) p.ops.push_back(rec(S_COMPUTE, ev_gemm(i)));
  }
  return p;
}

Plan build_reducescatter_plan_bidir(int n, int mode, bool two_halves, bool serial, bool fused) {
  Plan p;
  p.kind = 1;
  p.n = n;
  p.mode = mode;
  p.serial = serial || fused;
  p.fused = fused;
  p.bidir = true;
  serial = p.serial;
  const int KC = bidir_cw_len(n), KW = bidir_ccw_len(n);
  const int H = (two_halves && !fused) ? 2 : 1;
  p.n_events = 2 + 6 * n;
  auto ev_gemm = [&](int i, int h) { return 2 + 2 * i + h; };
  auto ev_arrive = [&](int i, int h) { return 2 + 2 * n + 2 * i + h; };
  auto ev_started = [&](int i, int h) { return 2 + 4 * n + 2 * i + h; };
  const StreamId cs = serial ? S_COMPUTE : S_COPY;
  // After GEMM(i, h): the cw accumulators move on unless the chain ended;
  // the ccw ones move after every partial, the last move being the epilogue
  // permute that brings them to the rank of their slice.
  auto cw_moves = [&](int i) { return i + 1 < KC; };
  auto ccw_moves = [&](int i) { return i < KW; };
  auto copy_exists = [&](int i) { return cw_moves(i) || ccw_moves(i); };
  auto prev_copy = [&](int i, int h, int* pi, int* ph) {
    if (h == 1) { *pi = i; *ph = 0; } else { *pi = i - 1; *ph = H - 1; }
    return *pi >= 0 && copy_exists(*pi);
  };
  const bool only_cw = (KW == 0);   // n == 1: the single GEMM writes the output

  for (int i = 0; i < KC; ++i) {
    const bool last_cw = (i == KC - 1);
    for (int h = 0; h < H; ++h) {
      if (!serial && i >= 1) p.ops.push_back(wait(S_COMPUTE, ev_arrive(i, h)));
      int pi, ph;
      if (!serial && prev_copy(i, h, &pi, &ph)) p.ops.push_back(hint_wait(S_COMPUTE, ev_started(pi, ph)));
      Op g;
      g.kind = OP_GEMM;
      g.stream = S_COMPUTE;
      g.iter = i;
      g.half = h;
      g.epi = (i == 0) ? EPI_STORE : EPI_ACCUM;
      g.final_store = only_cw;
      for (int r = 0; r < n; ++r) {
        Item it;
        it.rank = r;
        it.shard = rs_slice_cw(n, r, i);
        it.a = ref(B_A, r);
        it.b = ref(B_B, r);
        const BufRef acc = ref(B_ACC, r, i % 2, h);
        if (only_cw) it.c = ref(B_OUT, r, 0, h);
        else if (fused && !last_cw) it.c = ref(B_ACC, mod_n(r - 1, n), (i + 1) % 2, h);
        else it.c = acc;
        if (i > 0) {
          it.cin = acc;
          it.has_cin = true;
        }
        g.items.push_back(it);
      }
      if (i < KW) {
        for (int r = 0; r < n; ++r) {
          Item it;
          it.rank = r;
          it.shard = rs_slice_ccw(n, r, i);
          it.a = ref(B_A, r);
          it.b = ref(B_B, r);
          const BufRef acc = ref(B_ACC_CCW, r, i % 2, h);
          it.c = fused ? ref(B_ACC_CCW, mod_n(r + 1, n), (i + 1) % 2, h) : acc;
          if (i > 0) {
            it.cin = acc;
            it.has_cin = true;
          }
          g.items.push_back(it);
        }
      }
      p.ops.push_back(g);
      if (copy_exists(i) && !fused) {
        if (!serial) {
          p.ops.push_back(rec(S_COMPUTE, ev_gemm(i, h)));
          p.ops.push_back(wait(S_COPY, ev_gemm(i, h)));
          p.ops.push_back(rec(S_COPY, ev_started(i, h)));
        }
        Op c;
        c.kind = OP_COPY;
        c.stream = cs;
        c.iter = i;
        c.half = h;
        if (cw_moves(i)) {
          for (int r = 0; r < n; ++r) {
            Item it;
            it.rank = r;
            it.shard = rs_slice_cw(n, mod_n(r + 1, n), i);
            it.a = ref(B_ACC, mod_n(r + 1, n), i % 2, h);
            it.c = ref(B_ACC, r, (i + 1) % 2, h);
            c.items.push_back(it);
          }
        }
        if (ccw_moves(i)) {
          for (int r = 0; r < n; ++r) {
            Item it;
            it.rank = r;
            it.shard = rs_slice_ccw(n, mod_n(r - 1, n), i);
            it.a = ref(B_ACC_CCW, mod_n(r - 1, n), i % 2, h);
            it.c = ref(B_ACC_CCW, r, (i + 1) % 2, h);
            c.items.push_back(it);
          }
        }
        p.ops.push_back(c);
        if (!serial) p.ops.push_back(rec(S_COPY, ev_arrive(i + 1, h)));
      }
    }
  }
  // Align-and-sum: out[r] = cw[r] + ccw[r] (the ccw accumulator arrived with
  // the epilogue permute of iteration KW-1).
  if (!only_cw) {
    for (int h = 0; h < H; ++h) {
      // (With n odd, GEMM(KW, h) already waited for this arrival.)
      if (!serial && KW == KC) p.ops.push_back(wait(S_COMPUTE, ev_arrive(KW, h)));
      Op sm;
      sm.kind = OP_SUM;
      sm.stream = S_COMPUTE;
      sm.iter = KC;
      sm.half = h;
      sm.final_store = true;
      for (int r = 0; r < n; ++r) {
        Item it;
        it.rank = r;
        it.shard = r;
        it.a = ref(B_ACC, r, (KC - 1) % 2, h);
        it.cin = ref(B_ACC_CCW, r, KW % 2, h);
        it.has_cin = true;
        it.c = ref(B_OUT, r, 0, h);
        sm.items.push_back(it);
      }
      p.ops.push_back(sm);
    }
  }
  return p;
}

namespace {
bool same_buf(const BufRef& x, const BufRef& y) {
  return x.kind == y.kind && x.parity == y.parity && x.half == y.half && x.rank == y.rank;
}
}  // namespace

bool make_fine_grained(Plan& p, bool epilogue) {
  if (p.kind != 1) return false;
  if (p.bidir) {
    // Two-way ring: out[s] = cw[s] + ccw[s] is the consumer.  Only the fused
    // form has both last partials in the last launch (with copies, the ccw
    // one still has to travel).
    if (!p.fused) return false;
    bool any = false;
    for (size_t si = 0; si < p.ops.size(); ++si) {
      if (p.ops[si].kind != OP_SUM) continue;
      int last = -1;
      for (int k = static_cast<int>(si) - 1; k >= 0; --k)
        if (p.ops[k].kind == OP_GEMM) {
          last = k;
          break;
        }
      if (last < 0) return false;
      Op& g = p.ops[last];
      const Op sum = p.ops[si];
      for (const Item& o : sum.items) {
        int icw = -1, iccw = -1;
        for (int q = 0; q < static_cast<int>(g.items.size()); ++q) {
          if (same_buf(g.items[q].c, o.a)) icw = q;
          if (same_buf(g.items[q].c, o.cin)) iccw = q;
        }
        if (icw < 0) return false;   // the cw chain always ends in the last launch
        Item& cw = g.items[icw];
        cw.meet = cw.c;
        cw.c = o.c;
        cw.other = o.cin;
        cw.has_other = true;
        if (iccw >= 0) {
          Item& ccw = g.items[iccw];
          ccw.meet = ccw.c;
          ccw.c = o.c;
          ccw.other = o.a;
          ccw.has_other = true;
          cw.pair = iccw;
          ccw.pair = icw;
        }
      }
      g.epi = EPI_FINAL;
      g.final_store = true;
      p.ops.erase(p.ops.begin() + static_cast<std::ptrdiff_t>(si));
      --si;
      any = true;
    }
    return any;
  }
  // One-way ring: the last partial of each output is the only one in its
  // launch; with the fused epilogue as consumer it writes the output itself.
  if (!epilogue) return false;
  bool any = false;
  for (Op& o : p.ops) {
    if (o.kind != OP_GEMM || !o.final_store) continue;
    for (Item& it : o.items) {
      it.meet = it.c;
      it.pair = -1;
      it.has_other = false;
    }
    o.epi = EPI_FINAL;
    any = true;
  }
  return any;
}

namespace {

std::string bufname(const BufRef& b) {
  char s[64];
  switch (b.kind) {
    case B_LOOPED: std::snprintf(s, sizeof s, "looped%d", b.rank); break;
    case B_LOCAL: std::snprintf(s, sizeof s, "local%d", b.rank); break;
    case B_OUT: std::snprintf(s, sizeof s, "out%d.h%d", b.rank, b.half); break;
    case B_RECV: std::snprintf(s, sizeof s, "recv%d.p%d", b.rank, b.parity); break;
    case B_ACC: std::snprintf(s, sizeof s, "acc%d.p%d.h%d", b.rank, b.parity, b.half); break;
    case B_CASE2: std::snprintf(s, sizeof s, "c2acc%d", b.rank); break;
    case B_A: std::snprintf(s, sizeof s, "a%d", b.rank); break;
    case B_B: std::snprintf(s, sizeof s, "b%d", b.rank); break;
    case B_RECV_CCW: std::snprintf(s, sizeof s, "recvccw%d.p%d", b.rank, b.parity); break;
    case B_ACC_CCW: std::snprintf(s, sizeof s, "accccw%d.p%d.h%d", b.rank, b.parity, b.half); break;
    default: std::snprintf(s, sizeof s, "?%d", b.rank); break;
  }
  return s;
}

}  // namespace

std::string describe_plan(const Plan& p) {
  std::string out;
  char line[128];
  for (const Op& o : p.ops) {
    out += (o.stream == S_COMPUTE) ? "compute " : "copy ";
    switch (o.kind) {
      case OP_RECORD:
        std::snprintf(line, sizeof line, "record ev=%d\n", o.event);
        out += line;
        break;
      case OP_WAIT:
        std::snprintf(line, sizeof line, "wait ev=%d%s\n", o.event, o.hint ? " hint=1" : "");
        out += line;
        break;
      case OP_GEMM:
      case OP_COPY:
      case OP_SUM: {
        const char* kname = o.kind == OP_GEMM ? "gemm" : (o.kind == OP_COPY ? "copy" : "sum");
        std::snprintf(line, sizeof line, "%s it=%d h=%d epi=%d final=%d", kname, o.iter, o.half,
                      o.epi, o.final_store ? 1 : 0);
        out += line;
        // AllGather cases 1 and 3 write the slice of their shard: name it, so that
        // two items writing different slices of one output do not collide.
        const bool slice_out = p.kind == 0 && o.kind == OP_GEMM &&
                               (p.mode == CCE_AG_LHS_ROWS || p.mode == CCE_AG_RHS_COLS ||
                                p.mode == CCE_AG_LHS_BATCH);
        std::string rd, wr, sh, xs, prs;
        for (size_t q = 0; q < o.items.size(); ++q) {
          const Item& it = o.items[q];
          std::string ir = bufname(it.a), iw = bufname(it.c);
          if (slice_out && it.c.kind == B_OUT) iw += ".s" + std::to_string(it.shard);
          if (o.kind == OP_GEMM) ir += "+" + bufname(it.b);
          if (it.has_cin) ir += "+" + bufname(it.cin);
          if (it.has_fwd) iw += "+" + bufname(it.fwd);
          // EPI_FINAL: a paired item stores its partial at its meet buffer
          // when it claims the chunk first, and reads the pair's meet buffer
          // only after the pair's ready signal (listed under pairs=, not r=).
          if (o.kind == OP_GEMM && o.epi == EPI_FINAL) {
            if (it.pair >= 0) {
              iw += "+" + bufname(it.meet);
              if (static_cast<int>(q) < it.pair) {
                if (!prs.empty()) prs += ",";
                prs += std::to_string(q) + ":" + std::to_string(it.pair);
              }
            } else if (it.has_other) {
              ir += "+" + bufname(it.other);
            }
          }
          if (!rd.empty()) rd += ",";
          rd += ir;
          if (!wr.empty()) wr += ",";
          wr += iw;
          if (!xs.empty()) xs += ",";
          xs += ir + ">" + iw;
          if (!sh.empty()) sh += ",";
          sh += std::to_string(it.rank) + ":" + std::to_string(it.shard);
        }
        for (char& ch : rd) if (ch == '+') ch = ',';
        for (char& ch : wr) if (ch == '+') ch = ',';
        out += " r=" + rd + " w=" + wr + " x=" + xs + " shard=" + sh;
        if (!prs.empty()) out += " pairs=" + prs;
        out += "\n";
        break;
      }
    }
  }
  return out;
}

}  // namespace cce
