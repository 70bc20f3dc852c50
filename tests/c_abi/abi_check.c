/* A plain C consumer of the library's C ABI (include/taq.h): sizing and the
 * argument checks that run before any device work, so it needs no GPU.  Prints
 * one line per check and exits non-zero on the first mismatch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "taq.h"

static int fails = 0;

static void expect(const char* what, long got, long want) {
  printf("%s: %ld (want %ld)\n", what, got, want);
  if (got != want) ++fails;
}

int main(void) {
  static const uint8_t bits[2] = {8, 4};
  taq_kv_cache c;
  memset(&c, 0, sizeof(c));
  c.batch = 2;
  c.num_kv_heads = 2;
  c.head_dim = 128;
  c.group_size = 32;
  c.capacity = 256;
  c.layout = TAQ_LAYOUT_TOKEN;
  c.bits = bits;
  c.codes = (uint8_t*)(uintptr_t)0x10000;    /* never dereferenced */
  c.scales = (uint16_t*)(uintptr_t)0x20000;
  c.zeros = (uint8_t*)(uintptr_t)0x30000;

  expect("abi version positive", taq_abi_version() > 0, 1);
  /* per batch entry: 256 tokens x (128 + 64) code bytes */
  expect("codes bytes", (long)taq_kv_codes_bytes(&c), 2L * 256 * (128 + 64));
  expect("meta count", (long)taq_kv_meta_count(&c), 2L * 2 * 256 * 4);

  /* null input, then a range past the capacity, then a misaligned input */
  expect("quantize null x", taq_kv_quantize(&c, NULL, 0, 4, NULL), TAQ_ERR_INVALID_ARGUMENT);
  expect("error text set", taq_last_error()[0] != '\0', 1);
  expect("quantize past capacity",
         taq_kv_quantize(&c, (const void*)(uintptr_t)0x40000, 250, 7, NULL),
         TAQ_ERR_INVALID_ARGUMENT);
  expect("quantize misaligned", taq_kv_quantize(&c, (const void*)(uintptr_t)0x40002, 0, 4, NULL),
         TAQ_ERR_MISALIGNED);

  /* group size other than 32 */
  c.group_size = 16;
  expect("group 16", (long)taq_kv_codes_bytes(&c), 0);
  expect("quantize group 16", taq_kv_quantize(&c, (const void*)(uintptr_t)0x40000, 0, 4, NULL),
         TAQ_ERR_UNSUPPORTED);
  return fails ? 1 : 0;
}
