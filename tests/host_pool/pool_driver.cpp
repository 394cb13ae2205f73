// Drives the slot pool of csrc/pool.cpp on the CPU (built against the host
// stand-in of the HIP runtime in this folder) from a script on stdin, one
// operation per line, and prints one result line per operation.  The tests
// compare the results with the oracle's replay of the pool policy and check
// the slot bytes.  Test infrastructure.
//
//   init L E STRIDE CAPACITY   pinned store of L*E blobs (blob (l, e) byte i
//                              = (131 l + 17 e + 7 i) mod 256), pool
//   file PATH L E STRIDE CAPACITY   the same store as a container file
//   A l e1 e2 ...              acquire  -> "A ok s1 m1 s2 m2 ..." | "A err CODE"
//   R l e1 e2 ...              release  -> "R ok" | "R err CODE"
//   H l e1 e2 ...              prefetch -> "H ok LOADED" | "H err CODE"
//   E l e                      evict    -> "E ok" | "E err CODE"
//   F                          flush    -> "F ok" | "F err CODE"
//   S                          counters -> "S hits misses evictions prefetched bytes_h2d copies"
//   X l e                      slot     -> "X slot" (-1: not resident)
//   C l e                      slot bytes equal the store's blob -> "C 1" | "C 0"
//   P s                        slot s holds only 0xFF bytes -> "P 1" | "P 0"
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <sstream>
#include <string>
#include <vector>

#include "../../include/moe.h"

static uint8_t pattern(int l, int e, int64_t i) {
  return (uint8_t)((131 * l + 17 * e + 7 * i) & 0xFF);
}

int main() {
  expert_store* store = nullptr;
  slotpool* pool = nullptr;
  int64_t stride = 0;
  const uint8_t* base = nullptr;  // slot 0, learnt from the first acquire
  std::string line;
  char buf[1 << 16];
  while (std::fgets(buf, sizeof(buf), stdin)) {
    line = buf;
    std::istringstream in(line);
    std::string op;
    if (!(in >> op)) continue;
    if (op == "init" || op == "file") {
      std::string path;
      if (op == "file") in >> path;
      int L, E;
      long long cap;
      in >> L >> E >> stride >> cap;
      int32_t st = op == "init" ? expert_store_create(L, E, stride, &store)
                                : expert_store_open_file(path.c_str(), L, E, stride, 1, &store);
      if (st != MOE_OK) {
        std::printf("%s err %d %s\n", op.c_str(), st, moe_last_error());
        return 1;
      }
      std::vector<uint8_t> blob((size_t)stride);
      for (int l = 0; l < L; ++l)
        for (int e = 0; e < E; ++e) {
          for (int64_t i = 0; i < stride; ++i) blob[(size_t)i] = pattern(l, e, i);
          if (expert_store_write(store, l, e, blob.data(), stride) != MOE_OK) return 1;
        }
      st = slotpool_create(store, cap, 0, &pool);
      std::printf("%s %s\n", op.c_str(), st == MOE_OK ? "ok" : "err");
      if (st != MOE_OK) return 1;
    } else if (op == "H") {
      int l, e;
      in >> l;
      std::vector<int32_t> ex;
      while (in >> e) ex.push_back(e);
      int32_t loaded = -1;
      const int32_t st = slotpool_prefetch(pool, l, ex.data(), (int32_t)ex.size(), nullptr, &loaded);
      if (st == MOE_OK) std::printf("H ok %d\n", loaded);
      else std::printf("H err %d\n", st);
    } else if (op == "A" || op == "R") {
      int l;
      in >> l;
      std::vector<int32_t> ex;
      int e;
      while (in >> e) ex.push_back(e);
      if (op == "R") {
        const int32_t st = slotpool_release(pool, l, ex.data(), (int32_t)ex.size(), nullptr);
        if (st == MOE_OK) std::printf("R ok\n");
        else std::printf("R err %d\n", st);
        continue;
      }
      std::vector<const void*> ptrs(ex.size());
      std::vector<uint8_t> miss(ex.size());
      const int32_t st = slotpool_acquire(pool, l, ex.data(), (int32_t)ex.size(), nullptr,
                                          ptrs.data(), miss.data());
      if (st != MOE_OK) {
        std::printf("A err %d\n", st);
        continue;
      }
      std::printf("A ok");
      for (size_t i = 0; i < ex.size(); ++i) {
        int32_t slot = -1;
        slotpool_slot_of(pool, l, ex[i], &slot);
        const uint8_t* p = static_cast<const uint8_t*>(ptrs[i]);
        if (!base) base = p - (int64_t)slot * stride;
        if (p != base + (int64_t)slot * stride) {
          std::printf(" BADPTR\n");
          return 1;
        }
        std::printf(" %d %d", slot, (int)miss[i]);
      }
      std::printf("\n");
    } else if (op == "E") {
      int l, e;
      in >> l >> e;
      const int32_t st = slotpool_evict(pool, l, e);
      if (st == MOE_OK) std::printf("E ok\n");
      else std::printf("E err %d\n", st);
    } else if (op == "F") {
      const int32_t st = slotpool_flush(pool);
      if (st == MOE_OK) std::printf("F ok\n");
      else std::printf("F err %d\n", st);
    } else if (op == "S") {
      slotpool_counters c{};
      slotpool_stats(pool, &c);
      std::printf("S %lld %lld %lld %lld %lld %lld\n", (long long)c.hits, (long long)c.misses,
                  (long long)c.evictions, (long long)c.prefetched, (long long)c.bytes_h2d,
                  fake_hip_copies_of((size_t)stride));
    } else if (op == "X") {
      int l, e;
      in >> l >> e;
      int32_t slot = -1;
      slotpool_slot_of(pool, l, e, &slot);
      std::printf("X %d\n", slot);
    } else if (op == "C") {
      int l, e;
      in >> l >> e;
      int32_t slot = -1;
      slotpool_slot_of(pool, l, e, &slot);
      bool ok = slot >= 0 && base;
      for (int64_t i = 0; ok && i < stride; ++i) ok = base[(int64_t)slot * stride + i] == pattern(l, e, i);
      std::printf("C %d\n", ok ? 1 : 0);
    } else if (op == "P") {
      int s;
      in >> s;
      bool ok = base != nullptr;
      for (int64_t i = 0; ok && i < stride; ++i) ok = base[(int64_t)s * stride + i] == 0xFF;
      std::printf("P %d\n", ok ? 1 : 0);
    } else {
      std::printf("? %s\n", op.c_str());
      return 1;
    }
    std::fflush(stdout);
  }
  if (pool) slotpool_destroy(pool);
  if (store) expert_store_destroy(store);
  return 0;
}
