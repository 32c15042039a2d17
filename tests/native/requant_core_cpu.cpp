// Host build of the requantisation arithmetic (requant_core.h) for CPU
// tests: reads blocks from a binary file, writes codes and scale bytes.
// Input record per block: 16 code bytes, 2 scale bytes, 4-byte float gs.
// Output record: 16 code bytes, 1 scale byte.
#include <stdio.h>
#include <stdlib.h>
#include <vector>
#include "../../block_scaled_fp4_topk_amd/csrc/requant_core.h"

int main(int argc, char** argv) {
  if (argc != 3 && argc != 4) { fprintf(stderr, "usage: %s in out [tab]\n", argv[0]); return 2; }
  const bool tab = argc == 4;
  FILE* fi = fopen(argv[1], "rb");
  FILE* fo = fopen(argv[2], "wb");
  if (!fi || !fo) return 3;
  unsigned char rec[22];
  while (fread(rec, 1, 22, fi) == 22) {
    uint32_t c[4], o[4], sf;
    float gs;
    memcpy(c, rec, 16);
    sf = rec[16] | (rec[17] << 8);
    memcpy(&gs, rec + 18, 4);
    uint32_t b;
    if (tab) {
      float p1a, p3a, p1b, p3b;
      moefp4::rq::ro_pair(sf & 0xFF, fabsf(gs), p1a, p3a);
      moefp4::rq::ro_pair((sf >> 8) & 0xFF, fabsf(gs), p1b, p3b);
      b = moefp4::rq::requant_block_tab(c, sf, p1a, p3a, p1b, p3b,
                                        moefp4::rq::bits(gs) >> 31, o);
    } else {
      b = moefp4::rq::requant_block(c, sf, gs, o);
    }
    unsigned char out[17];
    memcpy(out, o, 16);
    out[16] = (unsigned char)b;
    fwrite(out, 1, 17, fo);
  }
  fclose(fi);
  fclose(fo);
  return 0;
}
