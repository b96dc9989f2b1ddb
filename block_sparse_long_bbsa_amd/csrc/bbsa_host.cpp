// Host-side query of the forward's work decomposition: for a call's shape,
// which work item every (workgroup, wavefront) of the attention kernel runs
// and which key blocks that item walks.  It runs the item mapping and the
// key-list construction of bbsa_schedule.h -- the code the kernels execute --
// on the host, so tests can check on a CPU that a launch covers every
// (batch, head, query tile, key block) of the pattern exactly once.
#include <stdint.h>

#include "bbsa.h"
#include "bbsa_schedule.h"

using namespace bbsa_sched;

extern "C" int bbsa_work_map(int B, int H, int L, int d, int block, int r, bbsa_dtype dtype, unsigned flags,
                             const int32_t *rand_attn, int32_t *records, int64_t capacity,
                             int64_t *count, int64_t *grid) {
  if (!count || !grid) return BBSA_ERR_ARG;
  // Stand-in device addresses: only their alignment is looked at.
  void *const fake = (void *)(uintptr_t)4096;
  Launch ln;
  const int st = setup_forward_ex(fake, fake, fake, nullptr, rand_attn, B, H, L, d, block, r, fake, nullptr,
                                  (int)dtype, flags, &ln);
  if (st < 0) return st;
  const Params &p = ln.p;
  const int waves = (dtype == BBSA_BF16) ? p.group : 1;
  int64_t n = 0;
  for (int64_t wg = 0; wg < ln.grid; ++wg) {
    for (int wv = 0; wv < waves; ++wv) {
      const Item u = decode_item(p, (int)wg, wv);
      if (u.bh >= p.bh_total) continue;
      if (records && n < capacity) {
        int32_t *rec = records + n * BBSA_WORK_RECORD_INTS;
        for (int i = 0; i < BBSA_WORK_RECORD_INTS; ++i) rec[i] = -1;
        rec[0] = (int32_t)wg;
        rec[1] = wv;
        rec[2] = 0;
        rec[3] = u.bh;
        rec[4] = u.qblock;
        rec[5] = u.qt;
        rec[6] = u.grow;
        rec[7] = u.chunk;
        int nblk = 0;
        int steps_per_block = 0;
        for (int lane = 0; lane < 64; ++lane) {
          int rnd = 0, rslot = -1;
          KeyWalk w = make_walk_base(p, u, lane, rnd, rslot);
          merge_plan(p, w, rnd, rslot);
          nblk = w.n_steps / w.steps_per_block;
          steps_per_block = w.steps_per_block;
          rec[16 + lane] = w.blk;
        }
        // The fp32 path splits a middle row's list into key parts.
        int pos0 = 0, pos1 = nblk;
        if (u.grow < 0 && p.mparts > 1) {
          pos0 = u.chunk * nblk / p.mparts;
          pos1 = (u.chunk + 1) * nblk / p.mparts;
        }
        rec[8] = pos0;
        rec[9] = pos1;
        rec[10] = steps_per_block;
        rec[11] = p.chunks;
        rec[12] = p.nparts;
        rec[13] = p.mparts;
        for (int lane = pos1; lane < 64; ++lane) rec[16 + lane] = -1;
        for (int lane = 0; lane < pos0; ++lane) rec[16 + lane] = -1;
      }
      ++n;
    }
  }
  *count = n;
  *grid = ln.grid;
  return st;
}
