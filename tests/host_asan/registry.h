// The buffers the sanitized host build's stand-in launches check against.
#pragma once
#include <cstddef>

void reg_clear();
void reg_add(const void *p, size_t bytes, const char *name);
int reg_failures();
int reg_launches();
