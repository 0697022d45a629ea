/* Part of the host sanitizer driver, in C because a C caller may pass any int
 * as a spear_status_t (C enums are ints; in C++ an out-of-range value of the
 * enum type would itself be undefined).  Declared here without the header, so
 * the parameter is a plain int, as the C ABI passes it. */
const char* spear_status_str(int status);

int spear_test_status_names(void) {
  for (int c = -5; c < 40; ++c) {
    const char* s = spear_status_str(c);
    if (!s || !s[0]) return 0;
  }
  return 1;
}
